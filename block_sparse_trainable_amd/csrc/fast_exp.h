// Exponential for softmax weights in VALU-bound loops.
#pragma once

#include <hip/hip_runtime.h>

namespace qsa {

// 2^x by the bare v_exp_f32.  It equals exp2f wherever exp2f's result is a
// normal number (x >= -126); below that the result, under 2^-126, may come
// back as 0 rather than a denormal, which no softmax sum whose largest term
// is 1 can register.  exp2f wraps the same instruction in five more (a
// range test, an offset and a rescale) to produce the denormals.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace qsa
