// Block-importance scoring (kernel b).
//
// "QSA (Qwen Sparse Attention)", Key math / How it works, (A): each query i
// scores each complete earlier block b as I_ib = sum over the indexer's query
// heads of ReLU(<q_i^h, k_b>), with block-causal masking (b < floor(p_i/r)).
// Output: one fp32 row of I per query, row stride W, entries b < c_i written.
//
// MFMA layout (v_mfma_f32_16x16x32_bf16, wave64).  The 16 rows of an A tile
// are (query, head) pairs ordered row = 4*query + head, the 16 columns of a B
// tile are blocks, and the contraction runs over the 128 dims in 4 k-steps.
// The accumulator of lane l holds rows 4*(l/16)+0..3 of column l%16, i.e.
// the four heads of one query for one block, so ReLU and the head sum happen
// in registers with no cross-lane traffic.  A and B fill each k-slot with the
// same dims, so the sum over k does not depend on the hardware's k order.
//
// Every kernel also leaves, per (query row, score segment), a 256-bin
// histogram of the scores it wrote (score_bin; u16 counts packed in pairs,
// accumulated in LDS and written once per workgroup), and zeroes the row's
// filter completion counter; the selection kernel reads both.
#include "qsa_common.h"

namespace qsa {
namespace {

__device__ __forceinline__ void hist_add(uint32_t* h, float v) {
  const uint32_t b = score_bin(__float_as_uint(v));
  atomicAdd(&h[b >> 1], 1u << ((b & 1u) << 4));
}

// The same for a score known to be >= +0.0 (sign bit clear), as every MFMA
// score is: its accumulation starts from +0.0, so a ReLU sum is never -0.0.
__device__ __forceinline__ void hist_add_nonneg(uint32_t* h, float v) {
  const int k = min(max((int)(__float_as_uint(v) >> 20) - 888, 0), kHistBins - 1);
  atomicAdd(&h[k >> 1], 1u + (uint32_t)(k & 1) * 65535u);
}

// Sum over a lane's four accumulator rows (the four indexer heads) of ReLU.
// ReLU as one integer max on the bit pattern: a float with the sign bit set
// is a negative int and becomes +0.0; every other value passes unchanged.
__device__ __forceinline__ float relu1(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}
__device__ __forceinline__ float relu_sum4(f32x4 a) {
  return relu1(a[0]) + relu1(a[1]) + relu1(a[2]) + relu1(a[3]);
}

struct ScoreOut {
  float* scores;      // [batch][nq_pad][W] f32 (16-bit keys for the streamed prefill rows)
  int64_t W;
  int64_t nq_pad;     // score rows per sequence (n_q rounded up for the prefill tiles)
  uint32_t* hist;     // [rows][n_sseg][kHistWords]
  int64_t n_sseg;
  uint32_t* done;     // [rows]
  int lr;             // log2 of the block size r
};

// ----------------------------------------------------------------- VALU ----
// Any dtype / head count: one workgroup per (query, 256 blocks), the query's
// heads staged in LDS as fp32.  Used for fp32 layers and non-MFMA layouts.
template <bool BF16>
__global__ __launch_bounds__(256) void score_valu_kernel(
    const void* __restrict__ q_idx_v, const int32_t* __restrict__ q_pos0, int n_q, int H,
    int D, const void* __restrict__ k_cmp_v, int64_t cap_blocks, ScoreOut o) {
  extern __shared__ float qs[];  // [H][D]
  __shared__ uint32_t hist[kHistWords];
  const int64_t row = blockIdx.x;
  const int s = (int)(row / n_q);
  const int j = (int)(row % n_q);
  const int64_t p = (int64_t)q_pos0[s] + j;
  const int64_t c = min(min(p >> o.lr, cap_blocks), o.W);
  if (blockIdx.y == 0 && threadIdx.x == 0) coherent_store(&o.done[row], 0u);
  for (int i = threadIdx.x; i < kHistWords; i += blockDim.x) hist[i] = 0u;
  for (int i = threadIdx.x; i < H * D; i += blockDim.x) {
    const int64_t off = row * H * D + i;
    qs[i] = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(q_idx_v)[off])
                 : static_cast<const float*>(q_idx_v)[off];
  }
  __syncthreads();
  const int64_t b = (int64_t)blockIdx.y * blockDim.x + threadIdx.x;
  if (b < c) {
    const int64_t kb = ((int64_t)s * cap_blocks + b) * D;
    float acc = 0.0f;
    for (int h = 0; h < H; ++h) {
      float dot = 0.0f;
      for (int d = 0; d < D; ++d) {
        const float kv = BF16 ? bf16_to_f32(static_cast<const uint16_t*>(k_cmp_v)[kb + d])
                              : static_cast<const float*>(k_cmp_v)[kb + d];
        dot = fmaf(qs[h * D + d], kv, dot);
      }
      acc += relu(dot);
    }
    o.scores[((int64_t)s * o.nq_pad + j) * o.W + b] = acc;
    hist_add(hist, acc);
  }
  __syncthreads();
  if ((int64_t)blockIdx.y < o.n_sseg)
    for (int i = threadIdx.x; i < kHistWords; i += blockDim.x)
      o.hist[hist_offset(row, blockIdx.y, o.n_sseg) + i] = hist[i];
}

// ------------------------------------------------------ MFMA, prefill ------
// Workgroup tile: 64 queries x one segment of blocks.  Wave w owns queries
// 16w..16w+15 (4 A row-tiles of 4 queries x 4 heads, kept in registers for
// the whole segment).  The segment is walked in chunks of 64 blocks; each
// chunk (64 x 256 B) is staged once in LDS, double-buffered, and read by all
// four waves as B tiles.  Block b of a chunk sits at LDS row
// 16 (b mod 4) + b / 4, so B tile t (rows 16t .. 16t + 15) holds blocks
// 4 l + t: after the chunk's four tiles each lane holds four consecutive
// blocks of a query, stored with one 8-byte write.
constexpr int kPQ = 64;       // queries per workgroup
constexpr int kChunk = 64;    // blocks per LDS chunk
constexpr int kRowB = 272;    // LDS bytes per block row (256 + 16 pad)

// HIST: also build the per-segment histograms (rows selected by the
// histogram-guided filter).  Without them the kernel fits three waves per SIMD.
template <bool HIST>
__global__ __launch_bounds__(256, HIST ? 2 : 3) void score_mfma_prefill_kernel(
    const uint16_t* __restrict__ q_idx, const int32_t* __restrict__ q_pos0, int n_q,
    const uint16_t* __restrict__ k_cmp, int64_t cap_blocks, int seg_blocks, ScoreOut o) {
  __shared__ __attribute__((aligned(16))) unsigned char lds[2][kChunk * kRowB];
  __shared__ uint32_t hist[HIST ? kPQ : 1][kHistWords];
  float* __restrict__ scores = o.scores;
  const int64_t W = o.W;
  const int s = blockIdx.z;
  // longest rows first: the last query tiles have the most blocks
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;

  const int j0 = qt * kPQ;
  const int j_last = min(j0 + kPQ, n_q) - 1;
  const int64_t pos0 = q_pos0[s];
  if (blockIdx.y == 0 && threadIdx.x < kPQ && j0 + (int)threadIdx.x < n_q)
    coherent_store(&o.done[(int64_t)s * n_q + j0 + threadIdx.x], 0u);
  const int64_t c_tile = min(min((pos0 + j_last) >> o.lr, cap_blocks), W);
  const int64_t b_lo = (int64_t)blockIdx.y * seg_blocks;
  const int64_t b_hi = min(b_lo + seg_blocks, c_tile);
  if (b_lo >= b_hi) return;  // no query of the tile reaches this segment
  if constexpr (HIST)
    for (int i = threadIdx.x; i < kPQ * kHistWords; i += 256) (&hist[0][0])[i] = 0u;

  // A operands: row tile rt covers queries j0 + 16w + 4rt + (0..3)
  u32x4 qa[4][4];
  int cq[4];        // candidate count of this lane's output query in each row tile
  uint32_t drow[4]; // that query's score row, at column 4 l16 (offset into scores)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int jq_a = j0 + 16 * wave + 4 * rt + (l16 >> 2);  // query of A row l16
    const int head = l16 & 3;
    const bool ok = jq_a < n_q;
    const uint16_t* src = q_idx + (((int64_t)s * n_q + (ok ? jq_a : 0)) * 4 + head) * 128 + 8 * gq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qa[rt][kk] = ok ? ld16(src + 32 * kk) : u32x4{0, 0, 0, 0};
    const int jq_o = j0 + 16 * wave + 4 * rt + gq;            // query of output rows 4gq..
    cq[rt] = jq_o < n_q ? (int)min(min((pos0 + jq_o) >> o.lr, cap_blocks), W) : 0;
    drow[rt] = (uint32_t)((jq_o - j0) * W + 4 * l16);
  }
  // The tile's rows (queries past n_q have padding rows of their own), so
  // every score store below is unconditional: a lane past its query's
  // candidates writes a slot the selection never reads.  Without HIST the
  // rows hold 16-bit keys: the top half of each score's bits, which orders
  // like the score (the selection resolves keys equal at its threshold from
  // exact recomputed scores).
  float* __restrict__ tile = scores + ((int64_t)s * o.nq_pad + j0) * W;
  uint16_t* __restrict__ tile16 =
      reinterpret_cast<uint16_t*>(scores) + ((int64_t)s * o.nq_pad + j0) * W;
  // Smallest candidate count among the wave's 16 queries (0 if any is past
  // n_q): chunks below it need no per-score mask.
  const int jw = j0 + 16 * wave;
  const int64_t c_wave = jw + 15 < n_q ? min(min((pos0 + jw) >> o.lr, cap_blocks), W) : 0;

  // cooperative chunk load: 1024 pieces of 16 B, four per thread, at 32-bit
  // offsets from the segment's first block
  const uint16_t* kseg = k_cmp + ((int64_t)s * cap_blocks + b_lo) * 128;
  const uint32_t last = (uint32_t)(b_hi - 1 - b_lo);
  auto load_chunk = [&](int64_t cb, u32x4 (&r)[4]) {
    const uint32_t c0 = (uint32_t)(cb - b_lo);
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t piece = threadIdx.x + 256u * u;
      const uint32_t blk = piece >> 4, col = piece & 15u;
      const uint32_t b = min(c0 + blk, last);   // blocks past b_hi score no query
      r[u] = ld16(kseg + (b * 128u + col * 8u));
    }
  };
  auto store_chunk = [&](int buf, const u32x4 (&r)[4]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int piece = threadIdx.x + 256 * u;
      const int blk = piece >> 4, col = piece & 15;
      const int lrow = 16 * (blk & 3) + (blk >> 2);
      *reinterpret_cast<u32x4*>(&lds[buf][lrow * kRowB + col * 16]) = r[u];
    }
  };
  uint32_t* hq[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) hq[rt] = hist[HIST ? 16 * wave + 4 * rt + gq : 0];

  u32x4 pre[4];
  load_chunk(b_lo, pre);
  store_chunk(0, pre);
  __syncthreads();
  int buf = 0;
  for (int64_t cb = b_lo; cb < b_hi; cb += kChunk) {
    const bool more = cb + kChunk < b_hi;
    if (more) load_chunk(cb + kChunk, pre);

    // two halves of 32 blocks: 8 accumulator tiles live at a time
    const bool full = !HIST || cb + kChunk <= c_wave;
    uint32_t k01[4];  // 16-bit keys of blocks 4 l16 and 4 l16 + 1, per row tile
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      f32x4 acc[4][2];
#pragma unroll
      for (int c2 = 0; c2 < 2; ++c2)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const u32x4 bv = *reinterpret_cast<const u32x4*>(
              &lds[buf][(32 * half + 16 * c2 + l16) * kRowB + 64 * kk + 16 * gq]);
#pragma unroll
          for (int rt = 0; rt < 4; ++rt)
            acc[rt][c2] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                as_bf16x8(qa[rt][kk]), as_bf16x8(bv),
                kk == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : acc[rt][c2], 0, 0, 0);
        }

      // epilogue: lane holds 4 heads of query (4rt + gq) for block 4 l16 + ct
#pragma unroll
      for (int rt = 0; rt < 4; ++rt) {
        float v[2];
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
          const int ct = 2 * half + c2;
          v[c2] = relu_sum4(acc[rt][c2]);
          if constexpr (HIST) {
            tile[drow[rt] + (uint32_t)cb + ct] = v[c2];
            if (full || cb + 4 * l16 + ct < cq[rt]) hist_add_nonneg(hq[rt], v[c2]);
          }
        }
        if constexpr (!HIST) {
          // the top halves of the two scores' bits, lower block first
          const uint32_t w = (__float_as_uint(v[0]) >> 16) | (__float_as_uint(v[1]) & 0xFFFF0000u);
          if (half == 0)
            k01[rt] = w;
          else
            *reinterpret_cast<uint2*>(tile16 + drow[rt] + (uint32_t)cb) = make_uint2(k01[rt], w);
        }
      }
    }
    if (more) {
      store_chunk(buf ^ 1, pre);
      __syncthreads();
      buf ^= 1;
    }
  }
  if constexpr (HIST) {
    __syncthreads();
    for (int i = threadIdx.x; i < kPQ * kHistWords; i += 256) {
      const int ql = i / kHistWords, w = i % kHistWords;
      if (j0 + ql < n_q)
        o.hist[hist_offset((int64_t)s * n_q + j0 + ql, blockIdx.y, o.n_sseg) + w] = hist[ql][w];
    }
  }
}

// ------------------------------------------------------- MFMA, decode ------
// Few queries, long rows: workgroup = (segment of WAVES*CPW*64 blocks, 4
// queries).  Each wave takes CPW 64-block chunks of the segment and issues
// all of their B-tile loads straight from HBM before its MFMAs (no reuse to
// stage through LDS); rows are 4 queries x 4 heads.
template <int WAVES, int CPW>
__global__ __launch_bounds__(64 * WAVES) void score_mfma_decode_kernel(
    const uint16_t* __restrict__ q_idx, const int32_t* __restrict__ q_pos0, int n_q,
    const uint16_t* __restrict__ k_cmp, int64_t cap_blocks, ScoreOut o) {
  constexpr int SEG = WAVES * CPW * 64;
  __shared__ uint32_t hist[4][kHistWords];
  float* __restrict__ scores = o.scores;
  const int64_t W = o.W;
  const int s = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int l16 = lane & 15;
  const int gq = lane >> 4;
  const int j0 = 4 * blockIdx.y;
  const int64_t pos0 = q_pos0[s];
  const int j_last = min(j0 + 4, n_q) - 1;
  if (blockIdx.x == 0 && threadIdx.x < 4 && j0 + (int)threadIdx.x < n_q)
    coherent_store(&o.done[(int64_t)s * n_q + j0 + threadIdx.x], 0u);
  const int64_t c_tile = min(min((pos0 + j_last) >> o.lr, cap_blocks), W);
  const int64_t seg_lo = (int64_t)blockIdx.x * SEG;
  const int64_t seg_hi = min(seg_lo + SEG, c_tile);
  if (seg_lo >= seg_hi) return;  // no query of the tile reaches this segment
  for (int i = threadIdx.x; i < 4 * kHistWords; i += 64 * WAVES) (&hist[0][0])[i] = 0u;
  __syncthreads();

  u32x4 qa[4];
  {
    const int jq_a = j0 + (l16 >> 2);
    const bool ok = jq_a < n_q;
    const uint16_t* src = q_idx + (((int64_t)s * n_q + (ok ? jq_a : 0)) * 4 + (l16 & 3)) * 128 + 8 * gq;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qa[kk] = ok ? ld16(src + 32 * kk) : u32x4{0, 0, 0, 0};
  }
  const int jq_o = j0 + gq;
  const int64_t cq = jq_o < n_q ? min(min((pos0 + jq_o) >> o.lr, cap_blocks), W) : 0;
  float* dst = scores + ((int64_t)s * o.nq_pad + (jq_o < n_q ? jq_o : 0)) * W;
  const uint16_t* kbase = k_cmp + (int64_t)s * cap_blocks * 128 + 8 * gq;

  // chunk c of this wave: blocks seg_lo + 64 * (c * WAVES + wave) .. +63
  // (adjacent waves stream adjacent memory)
  u32x4 kb[CPW][4][4];
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const int64_t b = seg_lo + 64 * (c * WAVES + wave) + 16 * ct + l16;
      const bool ok = b < seg_hi;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        kb[c][ct][kk] = ok ? ld16(kbase + b * 128 + 32 * kk) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
  for (int c = 0; c < CPW; ++c)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(qa[kk]), as_bf16x8(kb[c][ct][kk]),
                                                      acc, 0, 0, 0);
      const int64_t b = seg_lo + 64 * (c * WAVES + wave) + 16 * ct + l16;
      const float v = relu(acc[0]) + relu(acc[1]) + relu(acc[2]) + relu(acc[3]);
      if (b < cq) {
        dst[b] = v;
        hist_add(hist[gq], v);
      }
    }
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * kHistWords; i += 64 * WAVES) {
    const int ql = i / kHistWords, w = i % kHistWords;
    if (j0 + ql < n_q)
      o.hist[hist_offset((int64_t)s * n_q + j0 + ql, blockIdx.x, o.n_sseg) + w] = hist[ql][w];
  }
}

// Decode scoring shape: QSA_DEC_WAVES waves x QSA_DEC_CPW chunks per workgroup.
#ifndef QSA_DEC_WAVES
#define QSA_DEC_WAVES 8
#endif
#ifndef QSA_DEC_CPW
#define QSA_DEC_CPW 2
#endif
constexpr int kDecWaves = QSA_DEC_WAVES;
constexpr int kDecCpw = QSA_DEC_CPW;

}  // namespace

hipError_t launch_score(const Dims& d, const SelectPlan& pl, int batch, int n_q,
                        const void* q_idx, const int32_t* q_pos0, const void* k_cmp,
                        int64_t cap, void* workspace, hipStream_t st) {
  const int64_t cap_blocks = cap / d.r;
  char* ws = static_cast<char*>(workspace);
  ScoreOut o{reinterpret_cast<float*>(ws), pl.W, pl.nq_pad, reinterpret_cast<uint32_t*>(ws + pl.off_hist),
             pl.n_sseg, reinterpret_cast<uint32_t*>(ws + pl.off_done), d.lr};
  const unsigned segs = (unsigned)pl.n_sseg;
  if (pl.kernel == 1) {
    dim3 grid((unsigned)((n_q + kPQ - 1) / kPQ), segs, (unsigned)batch);
    if (pl.resident)
      hipLaunchKernelGGL(score_mfma_prefill_kernel<false>, grid, dim3(256), 0, st,
                         static_cast<const uint16_t*>(q_idx), q_pos0, n_q,
                         static_cast<const uint16_t*>(k_cmp), cap_blocks, (int)pl.sseg, o);
    else
      hipLaunchKernelGGL(score_mfma_prefill_kernel<true>, grid, dim3(256), 0, st,
                         static_cast<const uint16_t*>(q_idx), q_pos0, n_q,
                         static_cast<const uint16_t*>(k_cmp), cap_blocks, (int)pl.sseg, o);
  } else if (pl.kernel == 2) {
    dim3 grid(segs, (unsigned)((n_q + 3) / 4), (unsigned)batch);
    hipLaunchKernelGGL((score_mfma_decode_kernel<kDecWaves, kDecCpw>), grid, dim3(64 * kDecWaves), 0, st,
                       static_cast<const uint16_t*>(q_idx), q_pos0, n_q,
                       static_cast<const uint16_t*>(k_cmp), cap_blocks, o);
  } else {
    dim3 grid((unsigned)(batch * n_q), segs);
    const size_t shm = sizeof(float) * d.idx_heads * d.idx_dim;
    if (d.bf16)
      hipLaunchKernelGGL(score_valu_kernel<true>, grid, dim3(256), shm, st, q_idx, q_pos0, n_q,
                         d.idx_heads, d.idx_dim, k_cmp, cap_blocks, o);
    else
      hipLaunchKernelGGL(score_valu_kernel<false>, grid, dim3(256), shm, st, q_idx, q_pos0, n_q,
                         d.idx_heads, d.idx_dim, k_cmp, cap_blocks, o);
  }
  return hipGetLastError();
}

}  // namespace qsa
