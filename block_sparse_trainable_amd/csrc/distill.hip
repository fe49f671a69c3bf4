// Stage-1 indexer distillation: loss and gradients (qsa_indexer_distill), and
// the gradient back through the block compression (qsa_index_build_backward).
//
// "QSA (Qwen Sparse Attention)", Native trainability, stage 1: an indexer-only
// warm-up fits the indexer scores to a block-maxpooled version of the dense
// teacher attention distribution with a KL loss, while the model still runs
// dense attention.  The pages leave the details open; read as: for the query
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
// Kernels (one workgroup of 256 threads per query row unless noted):
//   teacher<PASS 1>  per head, the dense log-sum-exp over tokens 0..p;
//   teacher<PASS 2>  the head-averaged probabilities, max-pooled per block;
//   student          I_b, the loss terms, dI_b and dq_idx;
//   dk               one workgroup per (sequence, block): the rows whose
//                    candidates include the block form a contiguous range;
//   compress_bwd     one wave per block: back through RoPE, RMSNorm, mean.
#include <math.h>

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
  float* tb;       // [rows][W]    block maxima t_b, then dI_b
  float* ib;       // [rows][W]    I_b
  uint8_t* mk;     // [rows][W]    bit h: <q_idx^h, k_b> > 0
  int64_t W;       // row stride (candidates of the longest row, rounded up)
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
  const int r = 1 << lr;
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
      const int nb = kDT >> lr;   // blocks in this stretch (r <= 128 divides 256)
      if ((int)threadIdx.x < nb) {
        const int64_t b = (base >> lr) + threadIdx.x;
        if (b < c) {
          float mx = 0.0f;
          for (int u = 0; u < r; ++u) mx = fmaxf(mx, tt[threadIdx.x * r + u]);
          ws.tb[row * ws.W + b] = mx;
        }
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
  float* tb = ws.tb + row * ws.W;
  float* ib = ws.ib + row * ws.W;
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
    const float t = tb[b];
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
  // pass 2: dI_b over t_b in place
  const float invZ = c > 0 ? 1.0f / Z : 0.0f;
  for (int64_t b = threadIdx.x; b < c; b += kDT) tb[b] = expf(ib[b] - lseI) - tb[b] * invZ;
  __syncthreads();
  // dq_idx^h: thread (h, dims 2e, 2e+1), blocks in order
  const int h = threadIdx.x >> 6, e = threadIdx.x & 63;
  for (int hh = h; hh < H; hh += 4) {
    float d0 = 0.0f, d1 = 0.0f;
    for (int64_t b = 0; b < c; ++b) {
      const float w = ((mk[b] >> hh) & 1u) ? tb[b] : 0.0f;
      const int64_t ko = ((int64_t)s * cap_blocks + b) * 128 + 2 * e;
      d0 = fmaf(w, ldv<BF16>(k_cmp, ko), d0);
      d1 = fmaf(w, ldv<BF16>(k_cmp, ko + 1), d1);
    }
    dq_idx[(row * H + hh) * 128 + 2 * e] = d0;
    dq_idx[(row * H + hh) * 128 + 2 * e + 1] = d1;
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
    const float dI = ws.tb[row * ws.W + b];
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

DistillWs distill_layout(const Dims& d, int batch, int n_q, int32_t max_pos_end, void* base,
                         size_t* bytes) {
  DistillWs w{};
  w.W = score_row_width(d.r, max_pos_end);
  const size_t rows = (size_t)batch * n_q;
  auto al = [](size_t v) { return (v + 255) / 256 * 256; };
  size_t o = 0;
  const size_t o_lse = o; o = al(o + 4 * rows * (size_t)d.q_heads);
  const size_t o_tb = o;  o = al(o + 4 * rows * (size_t)w.W);
  const size_t o_ib = o;  o = al(o + 4 * rows * (size_t)w.W);
  const size_t o_mk = o;  o = al(o + rows * (size_t)w.W);
  if (bytes) *bytes = o;
  char* c = static_cast<char*>(base);
  if (c) {
    w.lse = reinterpret_cast<float*>(c + o_lse);
    w.tb = reinterpret_cast<float*>(c + o_tb);
    w.ib = reinterpret_cast<float*>(c + o_ib);
    w.mk = reinterpret_cast<uint8_t*>(c + o_mk);
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
#define QSA_DISTILL(BF)                                                                        \
  hipLaunchKernelGGL((distill_teacher_kernel<BF, 1>), dim3(rows), dim3(kDT), 0, st, q, k_cache, \
                     cap, n_q, q_pos0, d.q_heads, d.kv_heads, d.head_dim, d.scale, d.lr, ws);  \
  hipLaunchKernelGGL((distill_teacher_kernel<BF, 2>), dim3(rows), dim3(kDT), 0, st, q, k_cache, \
                     cap, n_q, q_pos0, d.q_heads, d.kv_heads, d.head_dim, d.scale, d.lr, ws);  \
  hipLaunchKernelGGL((distill_student_kernel<BF>), dim3(rows), dim3(kDT), 0, st, q_idx, k_cmp,  \
                     cap_blocks, n_q, q_pos0, cap, d.idx_heads, d.lr, ws, loss, dq_idx);      \
  hipLaunchKernelGGL((distill_dk_kernel<BF>), dim3((unsigned)(batch * nblk)), dim3(kDT), 0, st, \
                     q_idx, n_q, q_pos0, cap, d.idx_heads, d.lr, nblk, ws, dk_cmp, cap_blocks);
  if (d.bf16) {
    QSA_DISTILL(true)
  } else {
    QSA_DISTILL(false)
  }
#undef QSA_DISTILL
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
