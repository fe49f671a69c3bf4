// Internal declarations shared by the libqsa translation units: device
// helpers for gfx950 and the host-side launchers each kernel file exports to
// the C-ABI layer (qsa_api.hip).  Not part of the public interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qsa.h"

namespace qsa {

// ---------------------------------------------------------------- types ----
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------ bf16 conversions ----
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest, ties to even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// fp64 -> bf16 bits with a single rounding (nearest, ties to even): round
// the 52-bit mantissa to 7 bits in place; the result then converts to fp32
// exactly and its top half is the bf16 pattern.
__device__ __forceinline__ uint32_t f64_to_bf16(double x) {
  unsigned long long u = (unsigned long long)__double_as_longlong(x);
  const unsigned long long lsb = (u >> 45) & 1ull;
  u += 0xFFFFFFFFFFFull + lsb;           // (1 << 44) - 1 + lsb
  u &= ~((1ull << 45) - 1ull);
  const float f = (float)__longlong_as_double((long long)u);
  return __float_as_uint(f) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Ordering point for one wavefront: earlier LDS/global accesses of this wave
// are visible to its later accesses (used for per-wave LDS staging).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ float relu(float x) { return x > 0.0f ? x : 0.0f; }

// ------------------------------------------------- wave-level lane ops ----
// No LDS round trip: DPP row shifts and row broadcasts (inclusive scans over
// the 64 lanes; every lane must be active) and the gfx950 lane swaps
// (all-reduce over lanes l, l ^ 16, l ^ 32, l ^ 48).
__device__ __forceinline__ uint32_t wave_incl_add(uint32_t v) {
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}
__device__ __forceinline__ uint32_t wave_incl_max(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false));
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false));
  return v;
}
// Sum over each row of 16 lanes, left in the row's lane 15.
__device__ __forceinline__ float row16_sum_to_last(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x111, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x112, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x114, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x118, 0xF, 0xF, false));
  return v;
}
// x combined with the value of lane l ^ 16 (op(row 2r, row 2r+1) in both rows).
__device__ __forceinline__ float wave_max_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float wave_add_xor16(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float wave_add_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Cross-workgroup hand-off without cache maintenance.  A device-scope fence
// on this multi-XCD part writes back and invalidates the whole L2 of the
// issuing XCD; instead, data handed from one workgroup to another within a
// kernel is written and read with agent-scope relaxed atomics (coherent
// accesses that bypass the XCD-private L2 state), and ordered by waiting for
// the stores to complete before the completion counter is bumped.
template <class T>
__device__ __forceinline__ void coherent_store(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T coherent_load(const T* p) {
  return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Every store this workgroup made has completed (called by all threads,
// followed by a barrier, before one thread bumps the counter).
__device__ __forceinline__ void stores_complete() {
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
}
// Counter bump; returns true in the workgroup that arrives last.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t n) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == n - 1u;
}

// ------------------------------------------------- score histogram bins ----
// Scores are >= +0.0.  bin() maps a score's IEEE bits to one of 256 bins, 8
// per octave over [2^-16, 2^16) (exponent and top 3 mantissa bits), scores
// outside clamped to the end bins.  It is monotone non-decreasing in the
// score, which is all the selection relies on.
constexpr int kHistBins = 256;
constexpr int kHistWords = kHistBins / 2;  // two u16 counts per u32 word

__device__ __forceinline__ uint32_t score_bin(uint32_t bits) {
  if (bits & 0x80000000u) return 0u;      // never produced; treated as 0
  const int k = (int)(bits >> 20) - 888;  // 888 = 111 * 8: exponent of 2^-16
  return (uint32_t)min(max(k, 0), kHistBins - 1);
}

// Per-segment histogram slot of (row, segment): kHistWords u32 words.
__host__ __device__ inline int64_t hist_offset(int64_t row, int64_t seg, int64_t n_seg) {
  return (row * n_seg + seg) * kHistWords;
}

// --------------------------------------------------------- launch params ----
struct Dims {
  int r, lr, kB, idx_heads, idx_dim, rope_dims, q_heads, kv_heads, head_dim;  // r = 1 << lr
  bool bf16;
  float eps, scale;
  double base;
};

// Row width (floats) of the materialised score rows for queries ending
// before max_pos_end: the largest candidate count, rounded up to 4.
inline int64_t score_row_width(int r, int32_t max_pos_end) {
  int64_t c = max_pos_end > 0 ? (int64_t)(max_pos_end - 1) / r : 0;
  if (c < 1) c = 1;
  return (c + 3) / 4 * 4;
}

// Layout of the select workspace, derived from the call's sizes only.
//   scores  [batch][nq_pad][W] f32 block-importance rows (nq_pad >= n_q)
//   hist    [rows][n_sseg][128] u32 per-score-segment histograms (u16 pairs)
//   cand    [rows][kCandCap] u32x2 candidates of rows split over workgroups
//   done    [rows] u32             completion counters of split rows
struct SelectPlan {
  int kernel;        // 0 = VALU, 1 = MFMA prefill, 2 = MFMA decode
  int64_t W;         // score row width
  int64_t nq_pad;    // score rows per sequence
  bool resident;     // rows selected by one streaming pass: no histograms
  int64_t sseg;      // blocks per score segment
  int64_t n_sseg;
  int64_t fseg;      // score segments per filter workgroup
  int64_t n_fseg;    // filter workgroups per row
  size_t off_hist, off_slots, off_slotcnt, off_done, bytes;
};
constexpr int kCandCap = 4096;      // candidates a row may have (else fallback)
// blocks per score segment of the decode scoring kernel (waves x chunks x 64)
#ifndef QSA_DEC_WAVES
#define QSA_DEC_WAVES 8
#endif
#ifndef QSA_DEC_CPW
#define QSA_DEC_CPW 2
#endif
constexpr int64_t kDecodeScoreSeg = (int64_t)QSA_DEC_WAVES * QSA_DEC_CPW * 64;
SelectPlan select_plan(const struct Dims& d, int batch, int n_q, int32_t max_pos_end);

// ------------------------------------------------------------ launchers ----
// Each returns hipSuccess or the launch error; arguments are pre-validated.
hipError_t launch_compress(const Dims& d, int batch, const void* k_idx, int64_t cap,
                           const int32_t* len_before, const int32_t* len_after,
                           int max_new_blocks, const float* gain, void* k_cmp,
                           hipStream_t st);

hipError_t launch_score(const Dims& d, const SelectPlan& pl, int batch, int n_q,
                        const void* q_idx, const int32_t* q_pos0, const void* k_cmp,
                        int64_t cap, void* workspace, hipStream_t st);

hipError_t launch_select(const Dims& d, const SelectPlan& pl, int batch, int n_q,
                         const int32_t* q_pos0, int64_t cap, void* workspace, int32_t* sel,
                         int32_t* cnt, float* sel_scores, const void* q_idx, const void* k_cmp,
                         hipStream_t st);

// ------------------------------------------------------ fused decode step ----
// Score segments of 1024 blocks (a row's last segment also takes a remainder
// of up to 512 blocks), rows of up to kStepBmWords * 32 candidate blocks; a
// fixed control area at the start of the workspace holds, for up to
// kStepMaxBatch rows, each row's generation word, its scoring flags (one
// per segment) and split flags, its score-bin counts (two buffers, used in
// turn), and one error word.
constexpr int kStepSeg = 1024;
constexpr int kStepSegMax = kStepSeg + kStepSeg / 2;
constexpr int kStepBmWords = 8256;
constexpr int64_t kStepMaxBlocks = (int64_t)kStepBmWords * 32;       // 264,192
constexpr int kStepMaxBatch = 1024;
constexpr int kStepFaStride = 264;       // scoring flags per row (>= segments of a row)
constexpr int kStepFcStride = 32;        // split flags per row (>= attention splits)
constexpr int kStepOffGen = 0;           // control-area word offsets
constexpr int kStepOffErr = 2048;
constexpr int kStepOffFc = 4096;
constexpr int kStepOffFa = kStepOffFc + kStepMaxBatch * kStepFcStride;
constexpr int kStepOffAcc = kStepOffFa + kStepMaxBatch * kStepFaStride;  // [row][2][256]
constexpr size_t kStepCtlBytes = 4 * ((size_t)kStepOffAcc + (size_t)kStepMaxBatch * 2 * 256);

// Score segments of a row with c candidate blocks: 1024 each, the last one
// also holding a remainder of up to 512 (non-decreasing in c).
__host__ __device__ inline int step_nseg(int64_t c) {
  const int64_t full = c / kStepSeg, rem = c % kStepSeg;
  if (full == 0) return 1;
  return (int)((rem <= kStepSeg / 2) ? full : full + 1);
}
constexpr int kStepMaxSegs = (int)(kStepMaxBlocks / kStepSeg);        // 258

struct StepPlan {
  int64_t c_max;     // largest candidate count, floor((max_pos_end - 1) / r)
  int n_seg;         // score segments per row
  int n_split;       // attention splits per row
  size_t off_pairs, off_cum, off_part, bytes;
};
StepPlan step_plan(const Dims& d, int batch, int32_t max_pos_end);
bool decode_step_layout_ok(const Dims& d);
hipError_t launch_decode_step(const Dims& d, const StepPlan& pl, int batch, const void* q_idx,
                              const void* q, const void* k_idx, void* k_cmp, const float* gain,
                              const void* k_cache, const void* v_cache, int64_t cap,
                              const int32_t* q_pos, int32_t* sel, int32_t* cnt,
                              float* sel_scores, void* out, float* lse, void* workspace,
                              hipStream_t st);

// Attention workspace: the decode splits' partial states, or the prefill
// row order (MFMA path, 1,024 rows or more).
size_t attn_workspace_bytes(const Dims& d, int batch, int n_q, bool decode);

// Row order of a prefill-shaped call (one work item per query row): per
// row a sort key and the list index where its walk starts (-1: the
// position's own start), and, when row_order_sorts(), order[] = the rows
// grouped by the region their selection clusters in, then the rest in
// natural order.  key, first and order hold batch * n_q int32 each.
bool row_order_sorts(const Dims& d, int batch, int n_q);
hipError_t launch_row_order(const Dims& d, int batch, int n_q, const int32_t* q_pos0,
                            int64_t cap, const int32_t* sel, const int32_t* cnt, int32_t* key,
                            int32_t* first, int32_t* order, hipStream_t st);

// Attention backward: transposed index (per-block query lists) and per-head D.
hipError_t launch_offload_stage(const Dims& d, int batch, const int32_t* q_pos,
                                const int32_t* sel, const int32_t* cnt, const void* k_host_dev,
                                const void* v_host_dev, int64_t cap, void* hot_k, void* hot_v,
                                int32_t* hot_tag, int hot_units, void* stage_k, void* stage_v,
                                int64_t stage_tokens, int32_t* stage_sel, int32_t* stage_cnt,
                                int32_t* stage_pos, int32_t* stats, hipStream_t st);
size_t distill_workspace_bytes(const Dims& d, int batch, int n_q, int32_t max_pos_end);
hipError_t launch_distill(const Dims& d, int batch, int n_q, const void* q, const void* k_cache,
                          int64_t cap, const int32_t* q_pos0, int32_t max_pos_end,
                          const void* q_idx, const void* k_cmp, float* loss, float* dq_idx,
                          float* dk_cmp, void* workspace, hipStream_t st);
hipError_t launch_compress_backward(const Dims& d, int batch, const void* k_idx, int64_t cap,
                                    const int32_t* len_before, const int32_t* len_after,
                                    int max_new_blocks, const float* gain, const float* dk_cmp,
                                    float* dk_idx, hipStream_t st);

size_t bwd_workspace_bytes(const Dims& d, int batch, int n_q, int32_t max_pos_end);
hipError_t launch_attn_backward(const Dims& d, int batch, int n_q, const void* q,
                                const void* k_cache, const void* v_cache, int64_t cap,
                                const int32_t* q_pos0, int32_t max_pos_end, const int32_t* sel,
                                const int32_t* cnt, const void* out, const float* lse,
                                const void* dout, void* dq, float* dk, float* dv,
                                void* workspace, hipStream_t st);

hipError_t launch_attn(const Dims& d, int batch, int n_q, const void* q, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* q_pos0,
                       const int32_t* sel, const int32_t* cnt, void* out, float* lse,
                       void* workspace, bool decode, hipStream_t st);

}  // namespace qsa
