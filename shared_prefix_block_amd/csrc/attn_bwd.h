// Shared by the backward's two compilation units (attn_bwd.hip: preparation and dQ;
// attn_bwd_dkdv.hip: dK and dV): the kernels' parameter block, the rule that decides
// the precision of P and dS in the gradient products, and the dK/dV launcher.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "attn_common.h"
#include "psa_internal.h"

namespace psa {

struct BwdParams {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* nD;  // [hq, T]: -D = -sum_d dO * O (negated: dK/dV starts its dP sums from it)
  float* L2;  // [hq, T]
  const int32_t* end;   // interval form
  const int32_t* nkey;  // node form
  const int32_t* nlo;
  const int32_t* nw;
  int32_t causal;  // node form: 0 drops the kv <= q conjunct
  const int32_t* row_ptr;
  const int32_t* col;
  const uint8_t* kind;
  const int32_t* col_ptr;
  const int32_t* row;
  const uint8_t* kind_csc;
  const int32_t* qorder;
  const int32_t* korder;
  int64_t T;
  int32_t hq, hkv;
  float c;      // scale * log2(e)
  float scale;  // softmax scale
  int64_t n_work;
  int32_t chunk;
  int32_t c0;  // first output column of a launch that accumulates a column slice
};

// ---------------------------------------------------------------------------
// Precision of P and dS in the products that form dV, dK and dQ (bf16 inputs).
// kSplitAdaptive: a wave's fragment (16 queries x 32 keys) is rounded to bf16 once,
// unless its largest P exceeds kTauP or its largest |dS| exceeds kTauS; then the
// residual (frag_residual) goes through a second MFMA per product.  A rounded element
// is off by at most 2^-9 of itself, so a rounded fragment adds at most 2^-9 * tau per
// element times the other operand to a gradient, while the few large entries (rows
// that see few keys, where the softmax concentrates) keep about 16 bits.
// kSplitAll: every fragment gets the residual pass.  fp32 inputs have nothing to split.
// ---------------------------------------------------------------------------
constexpr int kSplitAdaptive = 0, kSplitAll = 1;
constexpr float kTauP = 0.125f, kTauS = 1.0f;

template <typename T, int MODE, bool WITH_P, bool WITH_S = true>
__device__ __forceinline__ bool split_wanted(const float* p8, const float* s8) {
  if constexpr (!std::is_same<T, bf16_t>::value) {
    return false;
  } else if constexpr (MODE == kSplitAll) {
    return true;
  } else {
    float mp = 0.f, ms = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      if constexpr (WITH_P) mp = fmaxf(mp, p8[j]);  // P >= 0
      if constexpr (WITH_S) ms = fmaxf(ms, fabsf(s8[j]));
    }
    return __any(mp > kTauP || ms > kTauS);  // wave-uniform
  }
}

// dK and dV of one backward (the launches of the dK/dV stage, p's work split and
// column slice set here); defined and instantiated in attn_bwd_dkdv.hip.
template <typename T, typename G, int D, int MODE, bool NODES>
hipError_t launch_dkdv_t(BwdParams p, int64_t n_ktiles, hipStream_t stream);

}  // namespace psa
