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
// an online softmax; each lane owns dimensions lane and lane + 64 of the output.  Everything a
// chunk reads is requested at once after its block ids: each lane's key row as 16-byte chunks,
// and for each of its dimensions the 8 consecutive keys of every 8-key group (contiguous in the V
// tile; a group's tile comes from its first lane).  Products and sums run in key and dimension
// order.
template <int DT_OUT, int D>
__device__ __forceinline__ void prefill_valu_part(const PrefillArgs& a, const int hq, const int row) {
  constexpr int E = 4;  // fp32 elements per 16-byte chunk of the K tile
  constexpr int NC = D / E;
  constexpr int DPL = (D + 63) / 64;
  const int g = hq / (a.Hq / a.Hkv);
  const int L = a.ctx_start + row + 1;  // keys this row sees
  const int lane = threadIdx.x;
  const float* __restrict__ kc = static_cast<const float*>(a.k);

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
    const int n = min(64, L - c0);
    int64_t tile = 0;
    if (valid) tile = (static_cast<int64_t>(min(max(a.table[t / kBlock], 0), a.num_blocks - 1)) * a.Hkv + g) * kBlock * D;
    u32x4 vr[8][DPL][2];
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      const int64_t gt = (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(tile >> 32), 8 * g8)) << 32) |
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tile), 8 * g8));
      const int half = ((c0 + 8 * g8) & 15) >> 3;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        vr[g8][k][0] = vr[g8][k][1] = u32x4{0, 0, 0, 0};
        if (8 * g8 < n && d < D) {
          const float* vb = static_cast<const float*>(a.v) + gt + (static_cast<int64_t>(half) * D + d) * 8;
          vr[g8][k][0] = *reinterpret_cast<const u32x4*>(vb);
          vr[g8][k][1] = *reinterpret_cast<const u32x4*>(vb + 4);
        }
      }
    }
    float sc = -INFINITY;
    if (valid) {
      const int off = t % kBlock;
      u32x4 kr[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) kr[c] = *reinterpret_cast<const u32x4*>(kc + tile + k_chunk_pos(off, c) * E);
      float acc = 0.f;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
#pragma unroll
        for (int e = 0; e < E; ++e) acc += qs[c * E + e] * __uint_as_float(kr[c][e]);
      }
      sc = acc;
    }
    const float m_new = fmaxf(m_run, wave_max64(sc));
    const float alpha = fast_exp2(m_run - m_new);
    const float pt = valid ? fast_exp2(sc - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum64(pt);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= alpha;
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      if (8 * g8 < n) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * g8 + e;
          const float pi = __shfl(pt, i);
          if (i < n) {
#pragma unroll
            for (int k = 0; k < DPL; ++k) {
              if (lane + 64 * k < D) o[k] += pi * __uint_as_float(vr[g8][k][e >> 2][e & 3]);
            }
          }
        }
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
