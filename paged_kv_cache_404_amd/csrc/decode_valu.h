// The vector-ALU decode body (any element type; the library uses it for fp32 caches), shared by
// the decode kernel (csrc/decode.hip) and the mixed decode + prefill launch (csrc/mixed.hip).
#pragma once

#include "decode_part.h"

namespace pkv {
namespace {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}

// Element e of a 16-byte chunk of DT elements, widened exactly to float.
template <int DT>
__device__ __forceinline__ float chunk_elem(const u32x4& w, int e) {
  if constexpr (DT == PKV_F32) {
    return __uint_as_float(w[e]);
  } else {
    const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
    return DT == PKV_BF16 ? bf16_bits_to_float(h) : f16_bits_to_float(h);
  }
}

// ------------------------------------------------------------------------------------------
// Vector-ALU body (any element type; used for fp32): query head hq, batch row yb, grid slice pz
// of a grid (Hq, B, max_parts); one wave.
// Lane i scores token c0 + i of each 64-token chunk, its row's 16-byte chunks requested at once;
// each lane owns dims lane and lane + 64 and reads them 8 tokens at a time (contiguous in the V
// tile), every group of the chunk requested before its sums.  Products and sums run in token and
// dimension order.
//
// Fused append (new_k set): token L - 1 takes its K/V from the input rows new_k / new_v in every
// workgroup that sees it, so no workgroup reads its cache slot; the workgroup of the KV head's
// first query head that owns the token's partition also copies the rows into the slot (when
// k_out is set), element for element, so the cache ends as an append would leave it.
// ------------------------------------------------------------------------------------------
template <int DT, int DT_OUT, int D>
__device__ __forceinline__ void decode_valu_part(const DecodeArgs& a, const int hq, const int yb, const int pz) {
  constexpr int ES = DT == PKV_F32 ? 4 : 2;  // element bytes
  constexpr int E = 16 / ES;                 // elements per 16-byte chunk of the K tile
  constexpr int NC = D / E;                  // chunks per token row
  constexpr int VW = ES / 2;                 // 16-byte loads per 8 tokens of one V dimension
  int b, p;
  work_item(a, yb, pz, b, p);
  const int G = a.Hq / a.Hkv;
  const int g = hq / G;
  const int L = clamp_len(a, b);
  const int pstart = p * a.part_size;
  if (pstart >= L) return;
  const int pend = min(pstart + a.part_size, L);
  const int nparts = (L + a.part_size - 1) / a.part_size;
  const int lane = threadIdx.x;
  const int32_t* table = a.tables + static_cast<int64_t>(b) * a.max_blocks;

  __shared__ float qs[D];
  for (int d = lane; d < D; d += 64)
    qs[d] = elem_to_float<DT>(a.q, (static_cast<int64_t>(b) * a.Hq + hq) * D + d) * a.scale_log2;
  __syncthreads();

  const bool fused = a.new_k != nullptr;
  const int tn = L - 1;                                    // the new token (fused append)
  const int64_t nrow = (static_cast<int64_t>(b) * a.Hkv + g) * D;  // its input rows
  if (fused && a.k_out != nullptr && hq % G == 0 && tn >= pstart && tn < pend) {
    const int64_t tile = (static_cast<int64_t>(clamp_blk(a, table[tn / kBlock])) * a.Hkv + g) * kBlock * D;
    const int off = tn % kBlock;
    for (int d = lane; d < D; d += 64) {
      copy_elem<DT>(a.k_out, tile + static_cast<int64_t>(k_chunk_pos(off, d / E)) * E + d % E, a.new_k, nrow + d);
      copy_elem<DT>(a.v_out, tile + static_cast<int64_t>((off >> 3) * D + d) * 8 + (off & 7), a.new_v, nrow + d);
    }
  }

  constexpr int DPL = (D + 63) / 64;  // dims per lane
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  __shared__ float sp[64];        // the chunk's weights

  for (int c0 = pstart; c0 < pend; c0 += 64) {
    const int t = c0 + lane;
    const bool valid = t < pend;
    const int n = min(64, pend - c0);
    int64_t tile = 0;
    if (valid) tile = (static_cast<int64_t>(clamp_blk(a, table[t / kBlock])) * a.Hkv + g) * kBlock * D;
    // The chunk's V: each lane's dimensions of every 8-token group, requested before the scores
    // (an 8-token group shares its block and half; its tile comes from the group's first lane).
    u32x4 vr[8][DPL][VW];
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      const int64_t gt = (static_cast<int64_t>(__builtin_amdgcn_readlane(static_cast<int>(tile >> 32), 8 * g8)) << 32) |
                         static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(tile), 8 * g8));
      const int half = ((c0 + 8 * g8) & 15) >> 3;
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
#pragma unroll
        for (int wv = 0; wv < VW; ++wv) vr[g8][k][wv] = u32x4{0, 0, 0, 0};
        if (8 * g8 < n && d < D) {
          const uint8_t* vb = static_cast<const uint8_t*>(a.v) + (gt + (static_cast<int64_t>(half) * D + d) * 8) * ES;
#pragma unroll
          for (int wv = 0; wv < VW; ++wv) vr[g8][k][wv] = *reinterpret_cast<const u32x4*>(vb + 16 * wv);
        }
      }
    }
    // Fused append: the new token's V elements of this lane's dimensions, requested with the rest.
    float nvv[DPL];
#pragma unroll
    for (int k = 0; k < DPL; ++k) {
      const int d = lane + 64 * k;
      nvv[k] = (fused && tn >= c0 && tn < c0 + n && d < D) ? elem_to_float<DT>(a.new_v, nrow + d) : 0.f;
    }
    float s = -INFINITY;
    if (valid) {
      const int off = t % kBlock;
      float acc = 0.f;
      if (fused && t == tn) {
        for (int d = 0; d < D; ++d) acc += qs[d] * elem_to_float<DT>(a.new_k, nrow + d);
      } else {
        // the token's row: D / E chunks of 16 bytes, all requested before the first product
        u32x4 kr[NC];
        const uint8_t* kb = static_cast<const uint8_t*>(a.k) + tile * ES;
#pragma unroll
        for (int c = 0; c < NC; ++c) kr[c] = *reinterpret_cast<const u32x4*>(kb + k_chunk_pos(off, c) * 16);
#pragma unroll
        for (int c = 0; c < NC; ++c) {
#pragma unroll
          for (int e = 0; e < E; ++e) acc += qs[c * E + e] * chunk_elem<DT>(kr[c], e);
        }
      }
      s = acc;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = fast_exp2(m_run - m_new);
    const float pt = valid ? fast_exp2(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(pt);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= alpha;
    sp[lane] = pt;
    __syncthreads();
    // Weighted sum, token by token in order: each lane's dimension d of 8 consecutive tokens is
    // 8 contiguous elements of the V tile ([half][D][8]).
#pragma unroll
    for (int g8 = 0; g8 < 8; ++g8) {
      if (8 * g8 < n) {
#pragma unroll
        for (int k = 0; k < DPL; ++k) {
          const int d = lane + 64 * k;
          if (d < D) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int i = 8 * g8 + e;
              if (i < n) {
                const float v = (fused && c0 + i == tn) ? nvv[k] : chunk_elem<DT>(vr[g8][k][e / E], e % E);
                o[k] += sp[i] * v;
              }
            }
          }
        }
      }
    }
    __syncthreads();  // the weights are rewritten by the next chunk
    m_run = m_new;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < D) emit<DT_OUT>(a, b, hq, p, nparts, d, D, m_run, l_run, o[k]);
  }
}

}  // namespace
}  // namespace pkv
