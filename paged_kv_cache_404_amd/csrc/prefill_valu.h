// The vector-ALU prefill body for fp32 caches, shared by the prefill kernel (csrc/prefill.hip) and
// the mixed decode + prefill launch (csrc/mixed.hip).
#pragma once

#include "prefill_tile.h"

namespace pkv {
namespace {

__device__ __forceinline__ float wave_max64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum64(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// fp32 caches: one wave per (query head hq, chunk row) on the vector ALU.  Lane i
// scores key c0 + i of each 64-key chunk of the row's visible keys 0 .. ctx_start + row and keeps
// an online softmax; each lane owns dimensions lane and lane + 64 of the output.
template <int DT_OUT, int D>
__device__ __forceinline__ void prefill_valu_part(const PrefillArgs& a, const int hq, const int row) {
  constexpr int E = 4;  // fp32 elements per 16-byte chunk of the K tile
  constexpr int DPL = (D + 63) / 64;
  const int g = hq / (a.Hq / a.Hkv);
  const int L = a.ctx_start + row + 1;  // keys this row sees
  const int lane = threadIdx.x;
  const float* __restrict__ kc = static_cast<const float*>(a.k);
  const float* __restrict__ vc = static_cast<const float*>(a.v);

  __shared__ float qs[D];
  for (int d = lane; d < D; d += 64)
    qs[d] = static_cast<const float*>(a.q)[(static_cast<int64_t>(row) * a.Hq + hq) * D + d] * a.scale_log2;
  __syncthreads();

  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  for (int c0 = 0; c0 < L; c0 += 64) {
    const int t = c0 + lane;
    const bool valid = t < L;
    int64_t tile = 0;
    int off = 0;
    float sc = -INFINITY;
    if (valid) {
      const int blk = min(max(a.table[t / kBlock], 0), a.num_blocks - 1);
      tile = (static_cast<int64_t>(blk) * a.Hkv + g) * kBlock * D;
      off = t % kBlock;
      float acc = 0.f;
      for (int d = 0; d < D; ++d) acc += qs[d] * kc[tile + static_cast<int64_t>(k_chunk_pos(off, d / E)) * E + d % E];
      sc = acc;
    }
    const float m_new = fmaxf(m_run, wave_max64(sc));
    const float alpha = fast_exp2(m_run - m_new);
    const float pt = valid ? fast_exp2(sc - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum64(pt);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= alpha;
    const int n = min(64, L - c0);
    for (int i = 0; i < n; ++i) {
      const float pi = __shfl(pt, i);
      const int64_t ti = __shfl(tile, i);
      const int oi = __shfl(off, i);
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < D) o[k] += pi * vc[ti + static_cast<int64_t>((oi >> 3) * D + d) * 8 + (oi & 7)];
      }
    }
    m_run = m_new;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < D) store_from_float<DT_OUT>(a.out, (static_cast<int64_t>(row) * a.Hq + hq) * D + d, o[k] / l_run);
  }
}

}  // namespace
}  // namespace pkv
