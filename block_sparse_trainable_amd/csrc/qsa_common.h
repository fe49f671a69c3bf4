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

// ------------------------------------------------- score histogram bins ----
// Scores are >= +0.0.  bin() maps a score's IEEE bits to one of 256 bins, 8
// per octave over [2^-16, 2^16) (exponent and top 3 mantissa bits), scores
// outside clamped to the end bins.  It is monotone non-decreasing in the
// score, which is all the selection relies on.
constexpr int kHistBins = 256;
constexpr int kHistWords = kHistBins / 2;  // two u16 counts per u32 word

__device__ __forceinline__ uint32_t score_bin(uint32_t bits) {
  const int k = (int)(bits >> 20) - 888;  // 888 = 111 * 8: exponent of 2^-16
  return (uint32_t)min(max(k, 0), kHistBins - 1);
}

// Per-segment histogram slot of (row, segment): kHistWords u32 words.
__host__ __device__ inline int64_t hist_offset(int64_t row, int64_t seg, int64_t n_seg) {
  return (row * n_seg + seg) * kHistWords;
}

// --------------------------------------------------------- launch params ----
struct Dims {
  int r, kB, idx_heads, idx_dim, rope_dims, q_heads, kv_heads, head_dim;
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
//   scores  [rows][W] f32          block-importance rows
//   hist    [rows][n_sseg][128] u32 per-score-segment histograms (u16 pairs)
//   slots   [rows][n_fseg][kSlotCap] u32x2 candidates of each filter segment
//   slotcnt [rows][n_fseg] u32
//   done    [rows] u32             filter-segment completion counters
struct SelectPlan {
  int kernel;        // 0 = VALU, 1 = MFMA prefill, 2 = MFMA decode
  int64_t W;         // score row width
  int64_t sseg;      // blocks per score segment
  int64_t n_sseg;
  int64_t fseg;      // scores per filter segment
  int64_t n_fseg;
  size_t off_hist, off_slots, off_slotcnt, off_done, bytes;
};
constexpr int kSlotCap = 1024;      // candidates one filter segment may hand over
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
                         int32_t* cnt, float* sel_scores, hipStream_t st);

// Decode attention workspace: [kAttnCounterRows] u32 completion counters
// (must be zero before the first call; every call leaves them zero), then
// the per-split partial states.
constexpr int64_t kAttnCounterRows = 65536;
size_t attn_workspace_bytes(const Dims& d, int rows, bool decode);

hipError_t launch_attn(const Dims& d, int batch, int n_q, const void* q, const void* k_cache,
                       const void* v_cache, int64_t cap, const int32_t* q_pos0,
                       const int32_t* sel, const int32_t* cnt, void* out, float* lse,
                       void* workspace, bool decode, hipStream_t st);

}  // namespace qsa
