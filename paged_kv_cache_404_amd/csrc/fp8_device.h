// Widening of OCP E4M3 codes to matrix-core operands, shared by the FP8 decode (csrc/fp8.hip) and
// the FP8 prefill tile (csrc/prefill_tile.h).  gfx950 converts two codes to two bf16 / fp16
// values in one v_cvt_scalef32_pk_{bf16,f16}_fp8 (scale 1: exact, every E4M3 value is a bf16 and
// an fp16 value).
#pragma once

#include "device.h"

namespace pkv {
namespace {

// Two E4M3 codes (the low or high half of w) -> two 16-bit elements of the product type, exact.
template <int DT, bool HIGH>
__device__ __forceinline__ uint32_t widen2(uint32_t w) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HIGH));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, HIGH));
  }
}

// Eight codes (two dwords) -> one 8-element operand fragment.
template <int DT>
__device__ __forceinline__ u32x4 widen8(uint32_t w0, uint32_t w1) {
  return u32x4{widen2<DT, false>(w0), widen2<DT, true>(w0), widen2<DT, false>(w1), widen2<DT, true>(w1)};
}

// Keep the first n (0..8) 16-bit elements of a fragment, zero the rest.
__device__ __forceinline__ u32x4 keep_first8(u32x4 v, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = (2 * w + 1 < n) ? 0xFFFFFFFFu : ((2 * w < n) ? 0x0000FFFFu : 0u);
    v[w] &= m;
  }
  return v;
}

}  // namespace
}  // namespace pkv
