// Stage-1 indexer distillation: loss and gradients (qsa_indexer_distill), and
// the gradient back through the block compression (qsa_index_build_backward).
//
// "QSA (Qwen Sparse Attention)", Native trainability, stage 1: before sparse
// training, only the indexer learns; its scores are pulled, by a KL
// divergence, toward the dense model's attention after a max over each
// block, and the model itself keeps attending densely meanwhile.  The pages
// leave the details open; read as: for the query
// at p, the teacher is the dense causal attention over tokens 0..p averaged
// over the main heads; its max over each candidate block's r tokens
// (b < c = floor(p/r)), renormalised over the candidates, is the target t;
// the student is softmax_b(I_b) over the same candidates; the loss is
// KL(t || softmax(I)), 0 when c = 0.  The teacher sends no gradient.  With
// Z = sum_b t_b of the unnormalised maxima,
//     loss = (sum_b t_b log t_b) / Z - log Z - (sum_b t_b I_b) / Z + logsumexp(I),
//     dL/dI_b = softmax(I)_b - t_b / Z,
//     dq_idx^h = sum_b dI_b [<q^h, k_b> > 0] k_b,
//     dk_b    += dI_b sum_h [<q^h, k_b> > 0] q^h        (ReLU'(0) = 0).
//
// Kernels.  bf16 layers with 16 query heads (teacher) and 4 indexer heads
// (student, key side) take the MFMA kernels; other layouts the VALU ones
// (one workgroup of 256 threads per query row unless noted):
//   teacher<PASS 1>  per head, the dense log-sum-exp over tokens 0..p;
//   teacher<PASS 2>  the head-averaged probabilities, max-pooled per 4-token
//                    unit (a block's target is the max over its units);
//   student          I_b, the loss terms, dI_b and dq_idx;
//   dk               one workgroup per (sequence, block) -- MFMA: per
//                    16-block tile: the rows whose candidates include the
//                    block form a contiguous range;
//   compress_bwd     one wave per block: back through RoPE, RMSNorm, mean.
#include <math.h>

#include "attn_tile.h"
#include "fast_exp.h"
#include "qsa_common.h"

namespace qsa {
namespace {

constexpr int kDT = 256;

template <bool BF16>
__device__ __forceinline__ float ldv(const void* p, int64_t i) {
  if constexpr (BF16) return bf16_to_f32(static_cast<const uint16_t*>(p)[i]);
  else return static_cast<const float*>(p)[i];
}

// Eight consecutive elements from a 16-byte (bf16) or 32-byte (fp32) aligned
// offset, as fp32.
template <bool BF16>
__device__ __forceinline__ void ld8(const void* p, int64_t i, float (&v)[8]) {
  if constexpr (BF16) {
    const u32x4 w = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p) + i);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = bf16_to_f32(w[e] & 0xFFFFu);
      v[2 * e + 1] = bf16_to_f32(w[e] >> 16);
    }
  } else {
    const float4 a = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i);
    const float4 b = *reinterpret_cast<const float4*>(static_cast<const float*>(p) + i + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
}

// Sum (or max) over the workgroup; every thread gets the result.
__device__ float wg_sum(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off);
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}
__device__ float wg_max(float v, float* red) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

struct DistillWs {
  float* lse;      // [rows][Hq]   teacher log-sum-exp per head
  float* um;       // [rows][Wu]   teacher maximum over each 4-token unit
  float* ib;       // [rows][W]    I_b, then dI_b
  uint8_t* mk;     // [rows][W]    bit h: <q_idx^h, k_b> > 0
  int64_t W;       // row stride (candidates of the longest row, rounded up to 16)
  int64_t Wu;      // row stride of um (4-token units below max_pos_end, rounded up)
  uint16_t* qT;    // [rows][128][4]  q_idx transposed (bf16, 4-head MFMA path)
  uint16_t* kT;    // [batch][nbt/4][128][4]  k_cmp in groups of 4 blocks (same)
  int64_t nbt;     // blocks per sequence covered by kT (a multiple of 16)
};

// ------------------------------------------------------------------ teacher --
// Thread per token; the scaled logits of every head for that token come from
// the query row in LDS.  PASS 1: per-thread online (max, sum) per head, then
// the workgroup's.  PASS 2: P_h = exp(logit - lse_h), the mean over heads, and
// the max over each block's r tokens (through LDS).
template <bool BF16, int PASS>
__global__ __launch_bounds__(kDT) void distill_teacher_kernel(
    const void* __restrict__ q, const void* __restrict__ kc, int64_t cap, int n_q,
    const int32_t* __restrict__ q_pos0, int Hq, int Hkv, int D, float scale, int lr,
    DistillWs ws) {
  __shared__ float qs[16 * 128];
  __shared__ float red[4];
  __shared__ float tt[kDT];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  if (PASS == 2 && c == 0) return;
  for (int i = threadIdx.x; i < Hq * D; i += kDT) qs[i] = ldv<BF16>(q, row * Hq * D + i);
  float lse[16];
  if constexpr (PASS == 2) {
#pragma unroll
    for (int h = 0; h < 16; ++h) lse[h] = h < Hq ? ws.lse[row * Hq + h] : 0.0f;
  }
  __syncthreads();
  const int HD = Hkv * D;
  const int G = Hq / Hkv;
  float m[16], l[16];
#pragma unroll
  for (int h = 0; h < 16; ++h) {
    m[h] = -INFINITY;
    l[h] = 0.0f;
  }
  const int64_t end = PASS == 1 ? p + 1 : (c << lr);   // pass 2: candidate blocks only
  for (int64_t base = 0; base < end; base += kDT) {
    const int64_t t = base + threadIdx.x;
    float mean = 0.0f;
    if (t < end) {
      const int64_t ko = ((int64_t)s * cap + t) * HD;
      float sd[16];
#pragma unroll
      for (int h = 0; h < 16; ++h) sd[h] = 0.0f;
      for (int g = 0; g < Hkv; ++g) {
        for (int d = 0; d < D; d += 8) {
          float kv[8];
          ld8<BF16>(kc, ko + g * D + d, kv);
#pragma unroll
          for (int h = 0; h < 16; ++h) {
            if (h < g * G || h >= (g + 1) * G) continue;
            float a = sd[h];
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaf(qs[h * D + d + e], kv[e], a);
            sd[h] = a;
          }
        }
      }
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h >= Hq) continue;
        const float x = sd[h] * scale;
        if constexpr (PASS == 1) {
          const float mn = fmaxf(m[h], x);
          l[h] = l[h] * expf(m[h] - mn) + expf(x - mn);
          m[h] = mn;
        } else {
          mean += expf(x - lse[h]);
        }
      }
    }
    if constexpr (PASS == 2) {
      tt[threadIdx.x] = mean / (float)Hq;
      __syncthreads();
      if ((int)threadIdx.x < kDT / 4) {
        const int64_t u = (base >> 2) + threadIdx.x;
        if (u < (c << (lr - 2)))
          ws.um[row * ws.Wu + u] =
              fmaxf(fmaxf(tt[4 * threadIdx.x], tt[4 * threadIdx.x + 1]),
                    fmaxf(tt[4 * threadIdx.x + 2], tt[4 * threadIdx.x + 3]));
      }
      __syncthreads();
    }
  }
  if constexpr (PASS == 1) {
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (h >= Hq) continue;   // uniform over the workgroup
      const float M = wg_max(m[h], red);
      const float L = wg_sum(m[h] == -INFINITY ? 0.0f : l[h] * expf(m[h] - M), red);
      if (threadIdx.x == 0) ws.lse[row * Hq + h] = M + logf(L);
    }
  }
}

// ------------------------------------------------------------ teacher, MFMA --
// bf16 layers with 16 query heads (the forward's MFMA shapes).  One workgroup
// of 8 waves per 16 consecutive query rows of a sequence; each wave owns 2 of
// them, i.e. 32 (query, head) columns = 2 MFMA column groups of 16: with Hkv
// KV heads a group holds Hkv queries x 16/Hkv heads of one KV head.  (Fewer
// queries per wave than 4 leave registers for two workgroups per CU, which
// hides more of each tile's latency than the halved K reuse costs.)  The queries sit in
// B-operand registers for the whole token loop; all eight waves share each
// 32-token K tile, staged in LDS (swizzled as the backward's K tile) and read
// as A operands: S^T = K_tile * Q per column group (v_mfma_f32_16x16x32_bf16).
// PASS 1 keeps an online (max, sum) per column in the log2 domain and writes
// lse per (row, head); PASS 2 turns the logits into probabilities, sums each
// (query, token)'s 16 heads across lanes, and writes the maximum of the head
// mean over each 4-token unit below the query's candidate limit.
// v plus its value in the lane the DPP control CTRL names (within a 16-lane
// row): a VALU add with a lane permutation, no LDS traffic
template <int CTRL>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

constexpr int kTW = 8;    // waves per teacher workgroup
constexpr int kTCG = 2;   // column groups (= query rows) per teacher wave

template <int HKV, int D, int PASS>
__global__ __launch_bounds__(64 * kTW) void distill_teacher_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ kc, int64_t cap, int n_q,
    const int32_t* __restrict__ q_pos0, float scale, int lr, DistillWs ws) {
  using S = MfmaShape<HKV, D>;
  constexpr int KD = S::KD, ROWB = S::ROWB, CH = S::CH, RPI = S::RPI;
  constexpr int G = 16 / HKV;          // heads per KV head
  constexpr int QPC = HKV;             // queries per column group
  constexpr int NKD = D / 32;          // k-steps over one KV head's dims
  constexpr int NCG = kTCG;            // column groups (= queries) per wave
  constexpr int QT = kTW * NCG;        // query rows per workgroup
  static_assert(NCG % HKV == 0, "a wave's columns must cover every KV head of its queries");
  __shared__ __attribute__((aligned(16))) unsigned char kbuf[3][32 * ROWB];   // a ring of three
  constexpr int NL = (32 / RPI) / kTW;   // tile loads per lane
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int tiles_per_seq = (n_q + QT - 1) / QT;
  const int s = blockIdx.x / tiles_per_seq;
  const int j0 = (blockIdx.x % tiles_per_seq) * QT;
  const int64_t pos0 = q_pos0[s];
  auto qpos = [&](int j) -> int64_t { return min(max(pos0 + j, (int64_t)0), cap - 1); };
  // token range of the tile
  const int jl = min(j0 + QT - 1, n_q - 1);
  const int64_t pmax = qpos(jl);
  const int64_t pmin = qpos(j0);   // positions grow with the row: every query sees tokens <= pmin
  const int64_t tok_end = PASS == 1 ? pmax + 1 : ((pmax >> lr) << lr);
  if (tok_end <= 0) return;
  // this lane's column in group cg: query qcol(cg), head hcol(cg); rows
  // past n_q stand in for the last row and write nothing.  Pass 1 with two
  // KV heads pairs the waves: wave w takes KV head w & 1 for the pair's 4
  // queries (group cg = queries 2cg, 2cg + 1 x that head's 8 heads), so both
  // of its groups use the same K fragments (half the LDS reads per score;
  // the per-head (max, sum) needs nothing from the other head).  Pass 2
  // sums all 16 heads of a query, so each wave keeps both KV heads there:
  // group cg = the wave's 2 queries x the 8 heads of KV head cg % HKV.
  constexpr bool PAIR = HKV == 2 && PASS == 1;
  static_assert(!PAIR || (NCG == 2 && kTW % 2 == 0), "wave pairs take 4 queries");
  const int gw = PAIR ? (wave & 1) : 0;   // the wave's KV head when paired
  auto qcol = [&](int cg) {
    return PAIR ? j0 + 4 * (wave >> 1) + 2 * cg + (l16 >> 3)
                : j0 + NCG * wave + (cg / HKV) * QPC + l16 / G;
  };
  auto hcol = [&](int cg) { return PAIR ? 8 * gw + (l16 & 7) : (cg % HKV) * G + l16 % G; };
  int32_t pq[NCG];   // positions (cap < 2^31)
  u32x4 qb[NCG][NKD];
  float lse2[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    const int jj = min(qcol(cg), jl);
    pq[cg] = (int32_t)qpos(jj);
    const int64_t row = (int64_t)s * n_q + jj;
#pragma unroll
    for (int kk = 0; kk < NKD; ++kk)
      qb[cg][kk] = ld16(q + (row * 16 + hcol(cg)) * D + 32 * kk + 8 * gq);
    if constexpr (PASS == 2) lse2[cg] = ws.lse[row * 16 + hcol(cg)] * kLog2e;
  }
  const float sl2 = scale * kLog2e;
  float m[NCG], l[NCG];
#pragma unroll
  for (int cg = 0; cg < NCG; ++cg) {
    m[cg] = -INFINITY;
    l[cg] = 0.0f;
  }
  static_assert(NL >= 1 && NL * kTW * RPI == 32, "tile loads must split evenly over the waves");
  const uint16_t* kbase = kc + (int64_t)s * cap * KD;
  // K rows of the tile at t0 into buffer bf (rows past tok_end read row 0, unused)
  auto load_tile = [&](int64_t t0, int bf) {
#pragma unroll
    for (int v = 0; v < NL; ++v) {
      const int u = wave + kTW * v;
      const int tk = RPI * u + lane / CH;
      const int chunk = (lane % CH) ^ (tk & 15);
      const int64_t tp = t0 + tk < tok_end ? t0 + tk : 0;
      __builtin_amdgcn_global_load_lds(
          (const __attribute__((address_space(1))) void*)(kbase + tp * KD + chunk * 8),
          (__attribute__((address_space(3))) void*)(kbuf[bf] + u * 1024), 16, 0, 0);
    }
  };
  // Tiles t and t + 32 are in flight when tile t is used.  A wave's loads
  // return in issue order, so once at most the next tile's NL are pending its
  // share of this tile has landed; the barrier then makes every wave's share
  // visible and, since every wave has left the previous tile, frees that
  // tile's buffer for the tile after next: one barrier per tile.
  load_tile(0, 0);
  if (32 < tok_end) load_tile(32, 1);
  int bf = 0;
  for (int64_t t0 = 0; t0 < tok_end; t0 += 32, bf = bf == 2 ? 0 : bf + 1) {
    if (t0 + 32 < tok_end)
      __builtin_amdgcn_s_waitcnt(NL | 0x70 | 0xF00);   // vmcnt(NL), expcnt/lgkmcnt any
    else
      __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t0 + 64 < tok_end) load_tile(t0 + 64, bf == 0 ? 2 : bf - 1);
    const unsigned char* kt = kbuf[bf];
    // S^T per column group and 16-token half
    f32x4 sa[NCG][2];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) sa[cg][0] = sa[cg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int tk = 16 * st + l16;
#pragma unroll
      for (int g = 0; g < (PAIR ? 1 : HKV); ++g)
#pragma unroll
        for (int kk = 0; kk < NKD; ++kk) {
          const int c0 = ((PAIR ? gw : g) * D + 32 * kk + 8 * gq) / 8;
          const u32x4 a = *reinterpret_cast<const u32x4*>(kt + tk * ROWB + ((c0 ^ (tk & 15)) * 16));
#pragma unroll
          for (int cg = PAIR ? 0 : g; cg < NCG; cg += PAIR ? 1 : HKV)
            sa[cg][st] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[cg][kk]),
                                                                 sa[cg][st], 0, 0, 0);
        }
    }
    if constexpr (PASS == 1) {
      if (t0 + 31 <= pmin) {
        // every token of the tile is visible to every query here.  Each
        // lane keeps its own (max, sum) over its tokens of the column; the
        // exponents are taken against the lane's running max as it stands,
        // and a tile sum above 2^64 (a logit more than 64 above that max, or
        // the first tile, max = -inf) is redone against the tile's max.  A
        // max taken from the lane's own logits keeps its largest term >= 1,
        // so terms lost to underflow are below 2^-126 of the sum, and sums
        // of terms <= 2^64 stay far from overflow.
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          float ps = 0.0f;
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) ps += exp2_fast(fmaf(sa[cg][st][i], sl2, -m[cg]));
          if (!(ps <= 0x1p64f)) {
            const float mt =
                fmaxf(fmaxf(fmaxf(sa[cg][0][0], sa[cg][0][1]), fmaxf(sa[cg][0][2], sa[cg][0][3])),
                      fmaxf(fmaxf(sa[cg][1][0], sa[cg][1][1]), fmaxf(sa[cg][1][2], sa[cg][1][3])));
            const float mn = fmaxf(m[cg], mt * sl2);   // the scale is positive
            ps = 0.0f;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 4; ++i) ps += exp2_fast(fmaf(sa[cg][st][i], sl2, -mn));
            l[cg] *= exp2_fast(m[cg] - mn);
            m[cg] = mn;
          }
          l[cg] += ps;
        }
      } else {
        const int32_t tb = (int32_t)t0 + 4 * gq;   // positions < cap < 2^31
#pragma unroll
        for (int cg = 0; cg < NCG; ++cg) {
          float x[2][4], mt = -INFINITY;
#pragma unroll
          for (int st = 0; st < 2; ++st)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              x[st][i] = tb + 16 * st + i <= pq[cg] ? sa[cg][st][i] * sl2 : -INFINITY;
              mt = fmaxf(mt, x[st][i]);
            }
          mt = wave_max_xor32(wave_max_xor16(mt));
          const float mn = fmaxf(m[cg], mt);
          if (mn != -INFINITY) {
            float ps = 0.0f;
#pragma unroll
            for (int st = 0; st < 2; ++st)
#pragma unroll
              for (int i = 0; i < 4; ++i) ps += exp2_fast(x[st][i] - mn);
            l[cg] = l[cg] * exp2_fast(m[cg] - mn) + ps;
            m[cg] = mn;
          }
        }
      }
    } else {
#pragma unroll
      for (int qs = 0; qs < NCG / HKV; ++qs) {
        float v[2][4];
#pragma unroll
        for (int st = 0; st < 2; ++st)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float a = 0.0f;
#pragma unroll
            for (int g = 0; g < HKV; ++g) {
              const int cg = qs * HKV + g;
              a += exp2_fast(fmaf(sa[cg][st][i], sl2, -lse2[cg]));
            }
            // sum over the query's heads held by the 8 (or 16) lanes of this
            // group: lane pairs xor 1 and xor 2 of each quad, then the two
            // quads of each 8-lane half (and the two halves of a row)
            a = dpp_add<0xB1>(a);    // quad_perm [1,0,3,2]
            a = dpp_add<0x4E>(a);    // quad_perm [2,3,0,1]
            a = dpp_add<0x141>(a);   // row_half_mirror
            if constexpr (HKV == 1) a = dpp_add<0x140>(a);   // row_mirror
            v[st][i] = a;   // the head sum; the mean's 1/16 is applied after the unit max
          }
        const int cg0 = qs * HKV;
        if (l16 % G == 0 && qcol(cg0) < n_q) {
          const int64_t row = (int64_t)s * n_q + qcol(cg0);
          const int64_t nu = ((int64_t)pq[cg0] >> lr) << (lr - 2);   // candidate units
#pragma unroll
          for (int st = 0; st < 2; ++st) {
            const int64_t u = (t0 + 16 * st + 4 * gq) >> 2;
            if (u < nu)
              ws.um[row * ws.Wu + u] =
                  fmaxf(fmaxf(v[st][0], v[st][1]), fmaxf(v[st][2], v[st][3])) * (1.0f / 16.0f);
          }
        }
      }
    }
  }
  if constexpr (PASS == 1) {
    // the four lanes of a column merge their (max, sum)
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) {
      const float M = wave_max_xor32(wave_max_xor16(m[cg]));
      const float lw = m[cg] == -INFINITY ? 0.0f : l[cg] * exp2_fast(m[cg] - M);
      const float lt = wave_add_xor32(wave_add_xor16(lw));
      if (gq == 0 && qcol(cg) < n_q)
        ws.lse[((int64_t)s * n_q + qcol(cg)) * 16 + hcol(cg)] = (M + log2f(lt)) * kLn2;
    }
  }
}

// ------------------------------------------------------------------ student --
template <bool BF16>
__global__ __launch_bounds__(kDT) void distill_student_kernel(
    const void* __restrict__ q_idx, const void* __restrict__ k_cmp, int64_t cap_blocks,
    int n_q, const int32_t* __restrict__ q_pos0, int64_t cap, int H, int lr, DistillWs ws,
    float* __restrict__ loss, float* __restrict__ dq_idx) {
  __shared__ float qs[16 * 128];
  __shared__ float red[4];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = min(max((int64_t)q_pos0[s] + j, (int64_t)0), cap - 1);
  const int64_t c = p >> lr;
  for (int i = threadIdx.x; i < H * 128; i += kDT) qs[i] = ldv<BF16>(q_idx, row * H * 128 + i);
  __syncthreads();
  const float* um = ws.um + row * ws.Wu;
  float* ib = ws.ib + row * ws.W;
  const int m4 = 1 << (lr - 2);   // 4-token units per block
  uint8_t* mk = ws.mk + row * ws.W;
  // pass 1: I_b, masks; online logsumexp of I; Z, sum t log t, sum t I
  float m = -INFINITY, l = 0.0f, z = 0.0f, a = 0.0f, bI = 0.0f;
  for (int64_t b = threadIdx.x; b < c; b += kDT) {
    const int64_t ko = ((int64_t)s * cap_blocks + b) * 128;
    float dots[16];
#pragma unroll
    for (int h = 0; h < 16; ++h) dots[h] = 0.0f;
    for (int d = 0; d < 128; d += 8) {
      float kv[8];
      ld8<BF16>(k_cmp, ko + d, kv);
#pragma unroll
      for (int h = 0; h < 16; ++h) {
        if (h >= H) continue;
        float acc = dots[h];
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(qs[h * 128 + d + e], kv[e], acc);
        dots[h] = acc;
      }
    }
    float I = 0.0f;
    uint32_t bits = 0;
#pragma unroll
    for (int h = 0; h < 16; ++h) {
      if (h < H && dots[h] > 0.0f) {
        I += dots[h];
        bits |= 1u << h;
      }
    }
    ib[b] = I;
    mk[b] = (uint8_t)bits;   // H <= 8 (validated)
    const float mn = fmaxf(m, I);
    l = l * expf(m - mn) + expf(I - mn);
    m = mn;
    float t = um[b * m4];
    for (int u = 1; u < m4; ++u) t = fmaxf(t, um[b * m4 + u]);
    z += t;
    if (t > 0.0f) a += t * logf(t);
    bI += t * I;
  }
  const float M = wg_max(m, red);
  const float L = wg_sum(m == -INFINITY ? 0.0f : l * expf(m - M), red);
  const float Z = wg_sum(z, red);
  const float A = wg_sum(a, red);
  const float BI = wg_sum(bI, red);
  const float lseI = M + logf(L);
  if (threadIdx.x == 0) loss[row] = c > 0 ? A / Z - logf(Z) - BI / Z + lseI : 0.0f;
  // pass 2: dI_b over I_b in place
  const float invZ = c > 0 ? 1.0f / Z : 0.0f;
  for (int64_t b = threadIdx.x; b < c; b += kDT) {
    float t = um[b * m4];
    for (int u = 1; u < m4; ++u) t = fmaxf(t, um[b * m4 + u]);
    ib[b] = expf(ib[b] - lseI) - t * invZ;
  }
  __syncthreads();
  // dq_idx^h: thread (h, dims 2e, 2e+1), blocks in order
  const int h = threadIdx.x >> 6, e = threadIdx.x & 63;
  for (int hh = h; hh < H; hh += 4) {
    float d0 = 0.0f, d1 = 0.0f;
    for (int64_t b = 0; b < c; ++b) {
      const float w = ((mk[b] >> hh) & 1u) ? ib[b] : 0.0f;
      const int64_t ko = ((int64_t)s * cap_blocks + b) * 128 + 2 * e;
      d0 = fmaf(w, ldv<BF16>(k_cmp, ko), d0);
      d1 = fmaf(w, ldv<BF16>(k_cmp, ko + 1), d1);
    }
    dq_idx[(row * H + hh) * 128 + 2 * e] = d0;
    dq_idx[(row * H + hh) * 128 + 2 * e + 1] = d1;
  }
}

// --------------------------------------------------------- student, MFMA --
// bf16 index rows, 4 indexer heads.  One wave per 4 consecutive query rows of
// a sequence (16 (query, head) columns: lane l16 = 4 query + head); blocks in
// tiles of 16.  Dots: C[block][column] = k_tile * q_idx^T
// (v_mfma_f32_16x16x32_bf16 over the 128 dims), so lane (column, gq) holds
// blocks 4gq .. 4gq+3 of its head; the head sum (I) and the mask bits meet
// across each lane quad, after which lane h of a quad takes the quad's block
// h, so each (query, block) pair is one lane's work.  Pass 1: the query's
// statistics (online logsumexp of I, Z, sum t log t, sum t I).  Pass 2
// recomputes the dots, forms dI, gathers the quad's four dI back to every
// lane and forms W = dI [dot > 0] -- the A-operand layout of a 16x16x16 MFMA
// over blocks -- and accumulates dq_idx = W * k (k in 4-block groups, kT),
// with W as bf16 hi + lo.  dI and the mask bytes go to the workspace for the key
// side; q_idx is also written transposed (qT) for it.
__device__ __forceinline__ float quad_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float quad_first(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x00, 0xF, 0xF, true));
}

typedef short bf16x4d __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x2p __attribute__((ext_vector_type(2)));
typedef float f32x2p __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_bf16(float x, float y) {   // nearest-even, one instruction
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2p{x, y}, bf16x2p));
}
__device__ __forceinline__ void split4(const float (&w)[4], bf16x4d& hi, bf16x4d& lo) {
  const uint32_t h0 = pk_bf16(w[0], w[1]), h1 = pk_bf16(w[2], w[3]);
  const uint32_t l0 = pk_bf16(w[0] - __uint_as_float(h0 << 16), w[1] - __uint_as_float(h0 & 0xFFFF0000u));
  const uint32_t l1 = pk_bf16(w[2] - __uint_as_float(h1 << 16), w[3] - __uint_as_float(h1 & 0xFFFF0000u));
  hi = __builtin_bit_cast(bf16x4d, make_uint2(h0, h1));
  lo = __builtin_bit_cast(bf16x4d, make_uint2(l0, l1));
}

__global__ __launch_bounds__(256) void distill_kt_kernel(const uint16_t* __restrict__ k_cmp,
                                                         int64_t cap_blocks, DistillWs ws) {
  const int s = blockIdx.y;
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;   // (block, dim)
  if (i >= ws.nbt * 128) return;
  const int64_t b = i >> 7;
  const int d = (int)(i & 127);
  const uint16_t v = b < cap_blocks ? k_cmp[((int64_t)s * cap_blocks + b) * 128 + d] : (uint16_t)0;
  ws.kT[(((int64_t)s * (ws.nbt / 4) + (b >> 2)) * 128 + d) * 4 + (b & 3)] = v;
}

// One workgroup of kSW waves per 4 kSW consecutive queries of a sequence; wave
// w takes queries 4w .. 4w+3 (16 A rows: query x head).  The candidate blocks
// are walked in chunks of kSC: each chunk's compressed keys (and, in pass 2,
// their transposed groups) are staged in LDS once for the workgroup, the
// next chunk's loads in flight meanwhile.
constexpr int kSW = 8;               // waves per student workgroup
constexpr int kSNT = 64 * kSW;
constexpr int kSQ = 4 * kSW;         // queries per student workgroup
constexpr int kSC = 64;              // blocks per LDS chunk
constexpr int kSP = 1024 / kSNT;     // 16-byte staging pieces per thread and array
constexpr int kSKRow = 256 + 16;     // LDS bytes per staged key row
constexpr int kSTG = 1024 + 128;     // LDS bytes per staged transposed group of 4 blocks

__global__ __launch_bounds__(kSNT) void distill_student_mfma_kernel(
    const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ k_cmp, int64_t cap_blocks,
    int batch, int n_q, const int32_t* __restrict__ q_pos0, int64_t cap, int lr, DistillWs ws,
    float* __restrict__ loss, float* __restrict__ dq_idx) {
  __shared__ __attribute__((aligned(16))) unsigned char kl[kSC * kSKRow];
  __shared__ __attribute__((aligned(16))) unsigned char tl[(kSC / 4) * kSTG];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int qn = l16 >> 2, h = l16 & 3;
  const int tiles = (n_q + kSQ - 1) / kSQ;
  const int s = (int)(blockIdx.x / (unsigned)tiles);
  const int j0 = (int)(blockIdx.x % (unsigned)tiles) * kSQ;
  const int jb = j0 + 4 * wave;
  const int j = jb + qn;
  const bool valid = j < n_q;
  const int64_t row = (int64_t)s * n_q + (valid ? j : n_q - 1);
  const int64_t p = min(max((int64_t)q_pos0[s] + (valid ? j : n_q - 1), (int64_t)0), cap - 1);
  const int64_t c = valid ? p >> lr : 0;
  // the workgroup's longest row is its last query's (positions grow with j)
  const int64_t cw = min(max((int64_t)q_pos0[s] + min(j0 + kSQ - 1, n_q - 1), (int64_t)0), cap - 1) >> lr;
  const int m4 = 1 << (lr - 2);
  u32x4 qb[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) qb[kk] = ld16(q_idx + (row * 4 + h) * 128 + 32 * kk + 8 * gq);
  if (valid) {   // q_idx transposed for the key side: qT[row][dim][head]
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e)
        ws.qT[(row * 128 + 32 * kk + 8 * gq + e) * 4 + h] =
            (uint16_t)(qb[kk][e >> 1] >> (16 * (e & 1)));
  }
  int64_t cmax = c;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1)
    cmax = max(cmax, (int64_t)__shfl_xor((long long)cmax, off));
  const uint16_t* kbase = k_cmp + (int64_t)s * cap_blocks * 128;
  const uint16_t* kT = ws.kT + (int64_t)s * (ws.nbt / 4) * 512;
  const int64_t last_group = ws.nbt / 4 - 1;
  const float* um = ws.um + row * ws.Wu;
  // chunk staging: 1024 pieces of 16 B for the keys (block, 16-byte column)
  // and 1024 for the transposed groups (group, 16-byte piece), kSP per thread
  auto load_k = [&](int64_t ch0, u32x4 (&r)[kSP]) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int piece = tid + kSNT * u;
      const int64_t b = min(ch0 + (piece >> 4), cap_blocks - 1);
      r[u] = ld16(kbase + b * 128 + (piece & 15) * 8);
    }
  };
  auto store_k = [&](const u32x4 (&r)[kSP]) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int piece = tid + kSNT * u;
      *reinterpret_cast<u32x4*>(&kl[(piece >> 4) * kSKRow + (piece & 15) * 16]) = r[u];
    }
  };
  auto load_t = [&](int64_t ch0, u32x4 (&r)[kSP]) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int piece = tid + kSNT * u;
      const int64_t g = min((ch0 >> 2) + (piece >> 6), last_group);
      r[u] = ld16(kT + g * 512 + (piece & 63) * 8);
    }
  };
  auto store_t = [&](const u32x4 (&r)[kSP]) {
#pragma unroll
    for (int u = 0; u < kSP; ++u) {
      const int piece = tid + kSNT * u;
      *reinterpret_cast<u32x4*>(&tl[(piece >> 6) * kSTG + (piece & 63) * 16]) = r[u];
    }
  };
  // dots of the chunk's tile at row t16: lane holds blocks t16 + 4gq + i for (qn, h)
  auto dots = [&](int t16, f32x4& acc) {
    acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&kl[(t16 + l16) * kSKRow + 64 * kk + 16 * gq]);
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(qb[kk]), acc, 0, 0, 0);
    }
  };
  auto target = [&](int64_t b) {
    float t = um[b * m4];
    for (int u = 1; u < m4; ++u) t = fmaxf(t, um[b * m4 + u]);
    return t;
  };
  // After the head sum the 4 lanes of a quad hold the same I for the tile's
  // blocks 4gq .. 4gq+3; lane h takes block 4gq + h, so each (query, block)
  // pair is handled by one lane.
  auto quad_sum4 = [&](const f32x4& acc, float (&Iq)[4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float I = fmaxf(acc[i], 0.0f);
      I += quad_xor1(I);
      I += quad_xor2(I);
      Iq[i] = I;
    }
  };
  auto pick = [&](const float (&v)[4]) {
    return h == 0 ? v[0] : h == 1 ? v[1] : h == 2 ? v[2] : v[3];
  };
  // ---- pass 1: statistics
  float m = -INFINITY, l = 0.0f, z = 0.0f, a = 0.0f, bI = 0.0f;
  u32x4 pk[kSP], pt[kSP];
  if (cw > 0) load_k(0, pk);
  for (int64_t ch0 = 0; ch0 < cw; ch0 += kSC) {
    __syncthreads();   // every wave is done with the previous chunk
    store_k(pk);
    __syncthreads();
    if (ch0 + kSC < cw) load_k(ch0 + kSC, pk);
#pragma unroll
    for (int t = 0; t < kSC / 16; ++t) {
      const int64_t b0 = ch0 + 16 * t;
      if (b0 >= cmax) break;
      f32x4 acc;
      dots(16 * t, acc);
      float Iq[4];
      quad_sum4(acc, Iq);
      const float I = pick(Iq);
      const int64_t b = b0 + 4 * gq + h;
      if (b < c) {
        const float mn = fmaxf(m, I);
        l = l * exp2_fast((m - mn) * kLog2e) + exp2_fast((I - mn) * kLog2e);
        m = mn;
        const float tv = target(b);
        z += tv;
        if (tv > 0.0f) a += tv * logf(tv);
        bI += tv * I;
      }
    }
  }
  // combine the 16 lanes of each query (its quad, and the four gq rows)
  {
    float M = fmaxf(m, quad_xor1(m));
    M = fmaxf(M, quad_xor2(M));
    M = wave_max_xor32(wave_max_xor16(M));
    l = (m == -INFINITY) ? 0.0f : l * exp2_fast((m - M) * kLog2e);
    m = M;
  }
  auto sum16 = [&](float v) {
    v += quad_xor1(v);
    v += quad_xor2(v);
    return wave_add_xor32(wave_add_xor16(v));
  };
  l = sum16(l);
  z = sum16(z);
  a = sum16(a);
  bI = sum16(bI);
  const float lseI = m + logf(l);
  if (valid && h == 0 && gq == 0) loss[row] = c > 0 ? a / z - logf(z) - bI / z + lseI : 0.0f;
  const float invZ = c > 0 ? 1.0f / z : 0.0f;
  // ---- pass 2: dI (one lane per pair), masks, dq_idx
  f32x4 dq[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) dq[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (cw > 0) {
    load_k(0, pk);
    load_t(0, pt);
  }
  for (int64_t ch0 = 0; ch0 < cw; ch0 += kSC) {
    __syncthreads();
    store_k(pk);
    store_t(pt);
    __syncthreads();
    if (ch0 + kSC < cw) {
      load_k(ch0 + kSC, pk);
      load_t(ch0 + kSC, pt);
    }
#pragma unroll
    for (int t = 0; t < kSC / 16; ++t) {
      const int64_t b0 = ch0 + 16 * t;
      if (b0 >= cmax) break;
      f32x4 acc;
      dots(16 * t, acc);
      float Iq[4], bitq[4];
      quad_sum4(acc, Iq);
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // the heads' mask bits of block 4gq + i, on every lane
        float bit = acc[i] > 0.0f ? (float)(1 << h) : 0.0f;
        bit += quad_xor1(bit);
        bit += quad_xor2(bit);
        bitq[i] = bit;
      }
      const int64_t b = b0 + 4 * gq + h;
      const float dI = b < c ? exp2_fast((pick(Iq) - lseI) * kLog2e) - target(b) * invZ : 0.0f;
      if (valid) {
        const int64_t o = row * ws.W + b;   // W is a multiple of 16
        ws.ib[o] = dI;
        ws.mk[o] = (uint8_t)pick(bitq);
      }
      // this lane's head over the quad's four blocks: W = dI [dot > 0]
      const float dIq[4] = {
          __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dI), 0x00, 0xF, 0xF, true)),
          __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dI), 0x55, 0xF, 0xF, true)),
          __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dI), 0xAA, 0xF, 0xF, true)),
          __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(dI), 0xFF, 0xF, 0xF, true))};
      float w[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = acc[i] > 0.0f ? dIq[i] : 0.0f;
      bf16x4d whi, wlo;
      split4(w, whi, wlo);
      const unsigned char* kt = tl + (4 * t + gq) * kSTG;
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const bf16x4d bk = __builtin_bit_cast(bf16x4d, *reinterpret_cast<const uint2*>(kt + (16 * db + l16) * 8));
        dq[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(whi, bk, dq[db], 0, 0, 0);
        dq[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wlo, bk, dq[db], 0, 0, 0);
      }
    }
  }
  // lane (dim 16db + l16, gq) holds (query gq, head i)
  if (jb + gq < n_q) {
    const int64_t orow = (int64_t)s * n_q + jb + gq;
#pragma unroll
    for (int db = 0; db < 8; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) dq_idx[(orow * 4 + i) * 128 + 16 * db + l16] = dq[db][i];
  }
}

// ------------------------------------------------------------ dk, MFMA --
// One workgroup per (sequence, 16-block tile); its waves take 4 query rows at
// a time from the rows that see the tile's first block.  A operand: lane
// (block, gq) holds W of query gq's 4 heads (dI and mask bytes from the
// student); B: q_idx transposed (qT), query gq's 4 heads at one dim; 16x16x16
// MFMAs contract over the 16 (query, head) pairs.  The waves meet in LDS.
__global__ __launch_bounds__(256) void distill_dk_mfma_kernel(
    int n_q, const int32_t* __restrict__ q_pos0, int64_t cap, int lr, int64_t ntile,
    DistillWs ws, float* __restrict__ dk_cmp, int64_t cap_blocks) {
  __shared__ float sd[16 * 128];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int l16 = lane & 15, gq = lane >> 4;
  const int s = (int)(blockIdx.x / ntile);
  const int64_t b0 = (blockIdx.x % ntile) * 16;
  const int64_t pos0 = q_pos0[s];
  const int64_t need = (b0 + 1) << lr;
  if (need > cap - 1) return;
  const int64_t j0 = max(need - pos0, (int64_t)0);
  if (j0 >= n_q) return;
  for (int i = threadIdx.x; i < 16 * 128; i += 256) sd[i] = 0.0f;
  f32x4 acc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db) acc[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int64_t b = b0 + l16;
  for (int64_t jg = j0 + 4 * wave; jg < n_q; jg += 16) {
    const int64_t jq = jg + gq;
    const bool vq = jq < n_q;
    const int64_t row = (int64_t)s * n_q + (vq ? jq : n_q - 1);
    const int64_t p = min(max(pos0 + (vq ? jq : n_q - 1), (int64_t)0), cap - 1);
    float w[4] = {0.f, 0.f, 0.f, 0.f};
    if (vq && b < (p >> lr)) {
      const float dI = ws.ib[row * ws.W + b];
      const uint32_t bits = ws.mk[row * ws.W + b];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) w[hh] = ((bits >> hh) & 1u) ? dI : 0.0f;
    }
    bf16x4d whi, wlo;
    split4(w, whi, wlo);
    const uint16_t* qt = ws.qT + row * 512;
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      uint2 qv = *reinterpret_cast<const uint2*>(qt + (16 * db + l16) * 4);
      if (!vq) qv = make_uint2(0u, 0u);
      const bf16x4d bq = __builtin_bit_cast(bf16x4d, qv);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(whi, bq, acc[db], 0, 0, 0);
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(wlo, bq, acc[db], 0, 0, 0);
    }
  }
  __syncthreads();   // LDS cleared
  // lane (dim 16db + l16, gq) holds blocks b0 + 4gq + i
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(&sd[(4 * gq + i) * 128 + 16 * db + l16], acc[db][i]);
  __syncthreads();
  for (int i = threadIdx.x; i < 16 * 128; i += 256) {
    const int64_t bb = b0 + (i >> 7);
    if (bb < cap_blocks) dk_cmp[((int64_t)s * cap_blocks + bb) * 128 + (i & 127)] += sd[i];
  }
}

// ----------------------------------------------------------------------- dk --
// One workgroup per (sequence, block b): the rows of the call whose query
// sees b (p >= r (b + 1)) are a contiguous range j >= j0.  Thread (row lane
// t >> 6, dims 2e, 2e+1); the four row lanes meet in LDS.
template <bool BF16>
__global__ __launch_bounds__(kDT) void distill_dk_kernel(
    const void* __restrict__ q_idx, int n_q, const int32_t* __restrict__ q_pos0, int64_t cap,
    int H, int lr, int64_t nblk, DistillWs ws, float* __restrict__ dk_cmp, int64_t cap_blocks) {
  __shared__ float part[4][128];
  const int s = (int)(blockIdx.x / nblk);
  const int64_t b = blockIdx.x % nblk;
  const int64_t pos0 = q_pos0[s];
  // j0: first row with min(pos0 + j, cap - 1) >= r (b + 1)
  const int64_t need = (b + 1) << lr;
  if (need > cap - 1) return;
  const int64_t j0 = max(need - pos0, (int64_t)0);
  if (j0 >= n_q) return;
  const int rl = threadIdx.x >> 6, e = threadIdx.x & 63;
  float d0 = 0.0f, d1 = 0.0f;
  for (int64_t jj = j0 + rl; jj < n_q; jj += 4) {
    const int64_t row = (int64_t)s * n_q + jj;
    const float dI = ws.ib[row * ws.W + b];
    const uint32_t bits = ws.mk[row * ws.W + b];
    for (int h = 0; h < H; ++h) {
      if (!((bits >> h) & 1u)) continue;
      const int64_t qo = (row * H + h) * 128 + 2 * e;
      d0 = fmaf(dI, ldv<BF16>(q_idx, qo), d0);
      d1 = fmaf(dI, ldv<BF16>(q_idx, qo + 1), d1);
    }
  }
  part[rl][2 * e] = d0;
  part[rl][2 * e + 1] = d1;
  __syncthreads();
  if (threadIdx.x < 128) {
    const int d = threadIdx.x;
    dk_cmp[((int64_t)s * cap_blocks + b) * 128 + d] +=
        part[0][d] + part[1][d] + part[2][d] + part[3][d];
  }
}

// ------------------------------------------------------------ compress bwd --
// One wave per block; lane l owns dims 2l, 2l+1 (as the forward).  In fp64:
// dy = RoPE_{-rb}(dk_b) (the transposed rotation), then
// dx = (g dy) / rms - x sum(g dy x) / (128 rms^3), and dx / r to each row.
template <bool BF16>
__global__ __launch_bounds__(kDT) void compress_bwd_kernel(
    const void* __restrict__ k_idx_v, int64_t cap, const int32_t* __restrict__ len_before,
    const int32_t* __restrict__ len_after, int max_new_blocks, const float* __restrict__ gain,
    double base, double eps, int rope_dims, const float* __restrict__ dk_cmp,
    float* __restrict__ dk_idx, int lr) {
  const int lane = threadIdx.x & 63;
  const int s = blockIdx.y;
  const int r = 1 << lr;
  const int64_t b0 = (int64_t)len_before[s] >> lr, b1 = (int64_t)len_after[s] >> lr;
  const int64_t cap_blocks = cap >> lr;
  const int d0 = 2 * lane;
  const int half = rope_dims / 2;
  int role = 0, partner = lane;
  double theta0 = 0.0, theta1 = 0.0;
  if (d0 < half) {
    role = 1;
    partner = lane + rope_dims / 4;
    theta0 = pow(base, -2.0 * (double)d0 / (double)rope_dims);
    theta1 = pow(base, -2.0 * (double)(d0 + 1) / (double)rope_dims);
  } else if (d0 < rope_dims) {
    role = 2;
    partner = lane - rope_dims / 4;
    theta0 = pow(base, -2.0 * (double)(d0 - half) / (double)rope_dims);
    theta1 = pow(base, -2.0 * (double)(d0 + 1 - half) / (double)rope_dims);
  }
  const double g0 = gain ? (double)gain[d0] : 1.0;
  const double g1 = gain ? (double)gain[d0 + 1] : 1.0;
  const int64_t stride = (int64_t)gridDim.x * (kDT / 64);
  for (int64_t b = b0 + (int64_t)blockIdx.x * (kDT / 64) + (threadIdx.x >> 6); b < b1;
       b += stride) {
    // x: the block mean (as the forward computes it)
    double x0 = 0.0, x1 = 0.0;
    const int64_t row0 = ((int64_t)s * cap + (b << lr)) * 128 + d0;
    for (int t = 0; t < r; ++t) {
      x0 += (double)ldv<BF16>(k_idx_v, row0 + t * 128);
      x1 += (double)ldv<BF16>(k_idx_v, row0 + t * 128 + 1);
    }
    x0 /= (double)r;
    x1 /= (double)r;
    double ss = x0 * x0 + x1 * x1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
    const double rms = sqrt(ss / 128.0 + eps);
    // dy = rotation by minus the angle of dk
    const int64_t kr = ((int64_t)s * cap_blocks + b) * 128 + d0;
    const double k0 = (double)dk_cmp[kr], k1 = (double)dk_cmp[kr + 1];
    const double o0 = __shfl(k0, partner), o1 = __shfl(k1, partner);
    double y0 = k0, y1 = k1;
    if (role != 0) {
      const double pos = (double)(b << lr);
      double s0, c0, s1, c1;
      sincos(pos * theta0, &s0, &c0);
      sincos(pos * theta1, &s1, &c1);
      if (role == 1) {   // forward: y_j = n_j c - n_{j+h} s  ->  transpose: + o s
        y0 = k0 * c0 + o0 * s0;
        y1 = k1 * c1 + o1 * s1;
      } else {           // forward: y_{j+h} = n_{j+h} c + n_j s  ->  transpose: - o s
        y0 = k0 * c0 - o0 * s0;
        y1 = k1 * c1 - o1 * s1;
      }
    }
    const double gy0 = g0 * y0, gy1 = g1 * y1;
    double dot = gy0 * x0 + gy1 * x1;
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) dot += __shfl_xor(dot, off);
    const double f = dot / (128.0 * rms * rms * rms);
    const float dx0 = (float)((gy0 / rms - x0 * f) / (double)r);
    const float dx1 = (float)((gy1 / rms - x1 * f) / (double)r);
    for (int t = 0; t < r; ++t) {
      dk_idx[row0 + t * 128] += dx0;
      dk_idx[row0 + t * 128 + 1] += dx1;
    }
  }
}

bool distill_student_mfma(const Dims& d) { return d.bf16 && d.idx_heads == 4 && d.idx_dim == 128; }

DistillWs distill_layout(const Dims& d, int batch, int n_q, int32_t max_pos_end, void* base,
                         size_t* bytes) {
  DistillWs w{};
  const int64_t cmax = max((int64_t)(max_pos_end - 1) >> d.lr, (int64_t)1);
  w.W = (cmax + 15) / 16 * 16;
  w.nbt = w.W;
  w.Wu = ((int64_t)max_pos_end / 4 + 3) / 4 * 4;
  const size_t rows = (size_t)batch * n_q;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t o = 0;
  const size_t o_lse = o; o = al(o + 4 * rows * (size_t)d.q_heads);
  const size_t o_um = o;  o = al(o + 4 * rows * (size_t)w.Wu);
  const size_t o_ib = o;  o = al(o + 4 * rows * (size_t)w.W);
  const size_t o_mk = o;  o = al(o + rows * (size_t)w.W);
  const bool m4 = distill_student_mfma(d);
  const size_t o_qt = o;  if (m4) o = al(o + rows * 128 * 4 * 2);
  const size_t o_kt = o;  if (m4) o = al(o + (size_t)batch * w.nbt * 128 * 2);
  if (bytes) *bytes = o;
  char* c = static_cast<char*>(base);
  if (c) {
    w.lse = reinterpret_cast<float*>(c + o_lse);
    w.um = reinterpret_cast<float*>(c + o_um);
    w.ib = reinterpret_cast<float*>(c + o_ib);
    w.mk = reinterpret_cast<uint8_t*>(c + o_mk);
    w.qT = reinterpret_cast<uint16_t*>(c + o_qt);
    w.kT = reinterpret_cast<uint16_t*>(c + o_kt);
  }
  return w;
}

}  // namespace

size_t distill_workspace_bytes(const Dims& d, int batch, int n_q, int32_t max_pos_end) {
  size_t b = 0;
  distill_layout(d, batch, n_q, max_pos_end, nullptr, &b);
  return b;
}

hipError_t launch_distill(const Dims& d, int batch, int n_q, const void* q, const void* k_cache,
                          int64_t cap, const int32_t* q_pos0, int32_t max_pos_end,
                          const void* q_idx, const void* k_cmp, float* loss, float* dq_idx,
                          float* dk_cmp, void* workspace, hipStream_t st) {
  const DistillWs ws = distill_layout(d, batch, n_q, max_pos_end, workspace, nullptr);
  const unsigned rows = (unsigned)(batch * n_q);
  const int64_t cap_blocks = cap >> d.lr;
  const int64_t nblk = max((int64_t)(max_pos_end - 1) >> d.lr, (int64_t)1);
  const bool mfma = d.bf16 && d.q_heads == 16 &&
                    ((d.kv_heads == 2 && (d.head_dim == 64 || d.head_dim == 128)) ||
                     (d.kv_heads == 1 && d.head_dim == 128));
  const unsigned qtiles = (unsigned)(batch * ((n_q + kTW * kTCG - 1) / (kTW * kTCG)));
#define QSA_TEACHER_MFMA(HKV, DD)                                                              \
  else if (d.kv_heads == HKV && d.head_dim == DD) {                                            \
    hipLaunchKernelGGL((distill_teacher_mfma_kernel<HKV, DD, 1>), dim3(qtiles), dim3(64 * kTW), 0, st, \
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache), \
                       cap, n_q, q_pos0, d.scale, d.lr, ws);                                  \
    hipLaunchKernelGGL((distill_teacher_mfma_kernel<HKV, DD, 2>), dim3(qtiles), dim3(64 * kTW), 0, st, \
                       static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k_cache), \
                       cap, n_q, q_pos0, d.scale, d.lr, ws);                                  \
  }
#define QSA_DISTILL(BF)                                                                        \
  if (!mfma) {                                                                                 \
    hipLaunchKernelGGL((distill_teacher_kernel<BF, 1>), dim3(rows), dim3(kDT), 0, st, q, k_cache, \
                       cap, n_q, q_pos0, d.q_heads, d.kv_heads, d.head_dim, d.scale, d.lr, ws); \
    hipLaunchKernelGGL((distill_teacher_kernel<BF, 2>), dim3(rows), dim3(kDT), 0, st, q, k_cache, \
                       cap, n_q, q_pos0, d.q_heads, d.kv_heads, d.head_dim, d.scale, d.lr, ws); \
  }                                                                                            \
  QSA_TEACHER_MFMA(2, 128)                                                                     \
  QSA_TEACHER_MFMA(1, 128)                                                                     \
  QSA_TEACHER_MFMA(2, 64)                                                                      \
  if (!smfma) {                                                                                \
    hipLaunchKernelGGL((distill_student_kernel<BF>), dim3(rows), dim3(kDT), 0, st, q_idx, k_cmp, \
                       cap_blocks, n_q, q_pos0, cap, d.idx_heads, d.lr, ws, loss, dq_idx);    \
    hipLaunchKernelGGL((distill_dk_kernel<BF>), dim3((unsigned)(batch * nblk)), dim3(kDT), 0, st, \
                       q_idx, n_q, q_pos0, cap, d.idx_heads, d.lr, nblk, ws, dk_cmp, cap_blocks); \
  }
  const bool smfma = distill_student_mfma(d);
  if (d.bf16) {
    QSA_DISTILL(true)
  } else {
    QSA_DISTILL(false)
  }
  if (smfma) {
    const int64_t ntile = ws.nbt / 16;
    hipLaunchKernelGGL(distill_kt_kernel, dim3((unsigned)((ws.nbt * 128 + 255) / 256), (unsigned)batch),
                       dim3(256), 0, st, static_cast<const uint16_t*>(k_cmp), cap_blocks, ws);
    const int64_t groups = (int64_t)batch * ((n_q + kSQ - 1) / kSQ);   // kSQ queries per workgroup
    hipLaunchKernelGGL(distill_student_mfma_kernel, dim3((unsigned)groups), dim3(kSNT),
                       0, st, static_cast<const uint16_t*>(q_idx),
                       static_cast<const uint16_t*>(k_cmp), cap_blocks, batch, n_q, q_pos0, cap,
                       d.lr, ws, loss, dq_idx);
    hipLaunchKernelGGL(distill_dk_mfma_kernel, dim3((unsigned)(batch * ntile)), dim3(256), 0, st,
                       n_q, q_pos0, cap, d.lr, ntile, ws, dk_cmp, cap_blocks);
  }
#undef QSA_DISTILL
#undef QSA_TEACHER_MFMA
  return hipGetLastError();
}

hipError_t launch_compress_backward(const Dims& d, int batch, const void* k_idx, int64_t cap,
                                    const int32_t* len_before, const int32_t* len_after,
                                    int max_new_blocks, const float* gain, const float* dk_cmp,
                                    float* dk_idx, hipStream_t st) {
  const int per = kDT / 64;
  const unsigned gx = (unsigned)min((int64_t)(max_new_blocks + per - 1) / per, (int64_t)65535);
  if (gx == 0) return hipSuccess;
  if (d.bf16)
    hipLaunchKernelGGL((compress_bwd_kernel<true>), dim3(gx, (unsigned)batch), dim3(kDT), 0, st,
                       k_idx, cap, len_before, len_after, max_new_blocks, gain, d.base,
                       (double)d.eps, d.rope_dims, dk_cmp, dk_idx, d.lr);
  else
    hipLaunchKernelGGL((compress_bwd_kernel<false>), dim3(gx, (unsigned)batch), dim3(kDT), 0, st,
                       k_idx, cap, len_before, len_after, max_new_blocks, gain, d.base,
                       (double)d.eps, d.rope_dims, dk_cmp, dk_idx, d.lr);
  return hipGetLastError();
}

}  // namespace qsa
