// One workgroup of paged decode attention on the matrix cores (bf16 / fp16), shared by the decode
// kernels (csrc/decode.hip) and the mixed decode + prefill launch (csrc/mixed.hip).  What is
// computed and how it maps onto the MI355X is described at the top of csrc/decode.hip.
#pragma once
#include "device.h"

namespace pkv {
namespace {

// Sequences a longest-first work order can name (it travels in the kernel arguments).
constexpr int kMaxOrder = 512;

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* tables;
  const int32_t* lens;
  float* part_ml;  // [B][Hq][max_parts][2] (m, l)
  float* part_o;   // [B][Hq][max_parts][D]
  int32_t Hq;
  int32_t Hkv;
  int32_t max_blocks;
  int32_t num_blocks;
  int32_t max_parts;
  int32_t part_size;  // tokens per partition, multiple of 16
  float scale_log2;   // scale * log2(e)
  const void* new_k;  // fused append: [B][Hkv][D] K/V of the token at position L - 1
  const void* new_v;
  void* k_out;        // fused append: the caches, written at that token's slot
  void* v_out;
  int32_t num_order;  // 0, or B: workgroup row y works on the sequence named by order[y]
  // Low 16 bits: the sequence; high 16 bits: a rotation r < max_parts of its partitions, grid
  // slice z working on partition (z + r) % max_parts.  Both only move work between workgroups.
  uint32_t order[kMaxOrder];
};

// The (sequence, partition) of grid row y, slice z.  The rotation is a bijection on
// [0, max_parts), so every partition is computed exactly once whatever the order says.
__device__ __forceinline__ void work_item(const DecodeArgs& a, int y, int z, int& b, int& p) {
  if (a.num_order) {
    const uint32_t o = a.order[y];
    b = static_cast<int>(o & 0xFFFFu);
    p = z + static_cast<int>(o >> 16);
    if (p >= a.max_parts) p -= a.max_parts;
  } else {
    b = y;
    p = z;
  }
}

// Zero the 16-bit elements i >= n of an 8-element fragment (n in [0, 8]).
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int n) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = (2 * w + 1 < n) ? 0xFFFFFFFFu : ((2 * w < n) ? 0x0000FFFFu : 0u);
    v[w] &= m;
  }
  return v;
}

// Context length and block ids come from device arrays the host cannot check without a sync.
// Out-of-contract values are clamped so that a bad input yields a wrong number, never a fault.
__device__ __forceinline__ int clamp_len(const DecodeArgs& a, int b) {
  return min(a.lens[b], min(a.max_parts * a.part_size, a.max_blocks * kBlock));
}
__device__ __forceinline__ int clamp_blk(const DecodeArgs& a, int blk) { return min(max(blk, 0), a.num_blocks - 1); }

// Writes the merged state of one (sequence, query head) partition: the final output when the
// sequence has a single partition, a partial otherwise.
template <int DT_OUT>
__device__ __forceinline__ void emit(const DecodeArgs& a, int b, int hq, int p, int nparts, int d, int D, float m,
                                     float l, float acc) {
  if (nparts == 1) {
    store_from_float<DT_OUT>(a.out, (static_cast<int64_t>(b) * a.Hq + hq) * D + d, acc / l);
  } else {
    const int64_t row = (static_cast<int64_t>(b) * a.Hq + hq) * a.max_parts + p;
    a.part_o[row * D + d] = acc;
    if (d == 0) {
      a.part_ml[row * 2] = m;
      a.part_ml[row * 2 + 1] = l;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Matrix-core kernel (bf16 / fp16).  grid = (Hkv, B, max_parts): the partition index varies
// slowest, so every sequence's full leading partitions are dispatched before the ragged last
// ones (longest work first, short work in the tail).  NW waves share one partition; wave w takes
// the 32-token steps w, w + NW, ...
//
// Memory pipeline: each wave keeps exactly one step of K/V in flight while it computes the
// previous one.  The next step's K fragments are loaded into the K registers as soon as the
// current Q.K products have consumed them, and the next V fragments right after P.V; only the
// last step of a wave is issued without a successor, so every wait inside the loop leaves the
// successor's loads outstanding.  The partition's block ids are loaded one per lane together with
// the context length (64 blocks per load), so a step's tile addresses come from a lane read.
// ------------------------------------------------------------------------------------------
//
// NEWTOK (fused append): the token at position L - 1 is this step's new token and its K/V come
// from the input rows new_k / new_v instead of the cache.  It lies in the sequence's last
// partition, in the last 32-token step of that partition; the wave that owns that step loads
// the new K/V straight into the operand layout and substitutes them for the cache slot's (stale)
// contents in its registers; it then stores the whole K and V tiles of that block (block
// table[(L - 1) / 16]) back, the new token at offset (L - 1) % 16 and every other slot with the
// bytes it was loaded with, so each cache line is written whole.  No other workgroup reads or
// writes that block (the last block of a sequence is private to it) in the same launch.
// LDS of one workgroup of the body below, in floats: the waves' partial outputs, maxima and sums.
template <int D, int G, int NW>
constexpr int decode_smem_floats() {
  return NW * G * D + 2 * NW * G;
}

// The body of one workgroup: KV head g, batch row yb (the sequence is order[yb] when a work order
// is given), grid slice pz (partition pz, rotated when a work order is given).  smem:
// decode_smem_floats<D, G, NW>() floats of LDS.
template <int DT, int DT_OUT, int D, int G, int NW, bool NEWTOK>
__device__ __forceinline__ void decode_mfma_part(const DecodeArgs& a, int g, int yb, int pz, float* smem) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  constexpr int KS = D / 32;        // k-steps of Q.K
  constexpr int NB = D / 16;        // 16-column blocks of P.V
  constexpr int TILE = kBlock * D;  // elements of one (block, head) tile
  constexpr int kTableSteps = 32;   // steps covered by one block-id load (64 blocks, one per lane)

  int b, p;
  work_item(a, yb, pz, b, p);
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int pstart = p * a.part_size;
  const int32_t* __restrict__ table = a.tables + static_cast<int64_t>(b) * a.max_blocks;
  // Issued before the length is known: its index is bounded by the table row, not by L.
  const int tab_first = table[min((pstart >> 4) + lane, a.max_blocks - 1)];
  const int L = clamp_len(a, b);
  if (pstart >= L) return;
  const int pend = min(pstart + a.part_size, L);
  const int nparts = (L + a.part_size - 1) / a.part_size;

  const int n16 = lane & 15;
  const int q4 = lane >> 4;
  const uint16_t* __restrict__ kc = static_cast<const uint16_t*>(a.k);
  const uint16_t* __restrict__ vc = static_cast<const uint16_t*>(a.v);
  const int nsteps = (pend - pstart + 31) >> 5;

  // Fused append: where the new token sits in the operand registers of its step (see the
  // token order below): K rows in lanes n16 == nk_lane (set nk_set), V elements nk_e of the
  // fragments in lanes q4 == nv_q4.
  const int last_st = nsteps - 1;
  const bool owner = NEWTOK && p == nparts - 1 && w == last_st % NW;
  const int nu = (L - 1) - (pstart + last_st * 32);  // index of the new token inside its step
  const int ntt = (L - 1) & 15;                     // offset inside its block
  const int nk_lane = (nu >> 4) * 8 + (ntt >> 3) * 4 + (ntt & 3);
  const int nk_set = (ntt >> 2) & 1;
  const int nv_q4 = (nu >> 4) * 2 + (ntt >> 3);
  u32x4 nk[KS];
  uint32_t nv[NB];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) nk[ks] = u32x4{0, 0, 0, 0};
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) nv[nb] = 0;
  if (owner) {
    const int64_t row = (static_cast<int64_t>(b) * a.Hkv + g) * D;
    const uint16_t* krow = static_cast<const uint16_t*>(a.new_k) + row;
    const uint16_t* vrow = static_cast<const uint16_t*>(a.new_v) + row;
    if (n16 == nk_lane) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) nk[ks] = *reinterpret_cast<const u32x4*>(krow + (4 * ks + q4) * 8);
    }
    if (q4 == nv_q4) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) nv[nb] = vrow[nb * 16 + n16];
    }
  }

  // Q^T fragments: lane (head n16, group q4) holds Q[head][ks*32 + 8*q4 .. +8]; padded heads are 0.
  u32x4 qf[KS];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(b) * a.Hq + g * G + min(n16, G - 1)) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = (n16 < G) ? *reinterpret_cast<const u32x4*>(qrow + ks * 32 + q4 * 8) : u32x4{0, 0, 0, 0};
    }
  }

  // Token order inside a 32-token step (blocks A = tokens 0..15, B = 16..31): Q.K product #s
  // (s = 0, 1) row m holds token 8*(m/4) + m%4 + 4s of block m/8 (the K tile order puts exactly
  // these rows of one k-step in one 512-byte run per block).  Lane (head, q4) then holds the
  // scores of step tokens 8*q4 .. 8*q4+7, the k-range its P row covers in P.V, whose V operand
  // (8 consecutive tokens of one dimension) is one 16-byte load from the V tile ([token half]
  // [D][8 tokens]: 16 lanes of one half read 256 contiguous bytes).
  const int k_in_tile = (q4 * 8 + (n16 & 7)) * 8;  // chunk (k-step 0, set 0) of this lane, in elements
  const bool k_from_b = n16 >= 8;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = (q4 & 1) * D * 8 + n16 * 8;

  f32x4 o[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY;  // reference maximum (log2 domain), meaningful in lanes n16 < G
  float l_run = 0.f;        // this lane's share of sum p

  for (int c0 = 0; c0 < nsteps; c0 += kTableSteps) {
    const int cend = min(nsteps, c0 + kTableSteps);
    int st = c0 + w;
    if (st >= cend) continue;
    const int cb0 = (pstart >> 4) + 2 * c0;                   // first block of this table chunk
    const int cnb = min(2 * kTableSteps, ((pend + 15) >> 4) - cb0);  // blocks of the chunk
    const int tab = clamp_blk(a, c0 == 0 ? tab_first : table[min(cb0 + lane, a.max_blocks - 1)]);

    u32x4 kf[2 * KS], vf[NB];
    auto tiles = [&](int s, int64_t& tA, int64_t& tB) {
      const int j = 2 * (s - c0);
      const int bA = __builtin_amdgcn_readlane(tab, j);
      const int bB = __builtin_amdgcn_readlane(tab, min(j + 1, cnb - 1));  // a lone last block pairs with itself
      tA = (static_cast<int64_t>(bA) * a.Hkv + g) * TILE;
      tB = (static_cast<int64_t>(bB) * a.Hkv + g) * TILE;
    };
    auto load_k = [&](int s) {
      int64_t tA, tB;
      tiles(s, tA, tB);
      const uint16_t* kp = kc + (k_from_b ? tB : tA) + k_in_tile;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (2 * ks) * 256));
        kf[KS + ks] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kp + (2 * ks + 1) * 256));
      }
    };
    auto load_v = [&](int s) {
      int64_t tA, tB;
      tiles(s, tA, tB);
      const uint16_t* vp = vc + (v_from_b ? tB : tA) + v_in_tile;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        vf[nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + nb * 16 * 8));
    };

    // One 32-token step; with `prefetch` the successor's loads are issued as registers free up.
    // The empty asm statements keep those loads where they are written.
    auto step = [&](int s, const bool prefetch) {
      const int nvalid = min(32, pend - (pstart + s * 32));
      const bool new_step = !prefetch && owner && s == last_st;
      // The new token's block (step block A or B) and its tile offset, for the store-back.
      const bool in_b = (nu >> 4) != 0;
      if (new_step) {
        // The new token replaces what its cache slot held before this launch.  The last step of
        // a wave is always the one issued without a successor.  The asm operands keep the
        // compiler from consuming (and so waiting for) the new token's loads before this step.
        // K is substituted here, V just before the P.V product, so this step still waits for
        // its V tile no earlier than any other step.
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(nk[ks]));
        if (n16 == nk_lane) {
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (nk_set) {
              kf[KS + ks] = nk[ks];
            } else {
              kf[ks] = nk[ks];
            }
          }
        }
        // The registers now hold the new token's K (the other slots as loaded).  Its bytes lie
        // in the half of the tile that holds its 4-token set (token order above): those 16 lines
        // (8 tokens each, one 16-byte chunk of each) are stored back with the load's own lane
        // pattern, so every line written is written whole.  Without k_out the caller writes the
        // cache itself (paged_attention_decode_newest).
        if (a.k_out != nullptr && k_from_b == in_b) {
          int64_t tA, tB;
          tiles(s, tA, tB);
          uint16_t* kp = static_cast<uint16_t*>(a.k_out) + (in_b ? tB : tA) + k_in_tile + nk_set * 256;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
            *reinterpret_cast<u32x4*>(kp + (2 * ks) * 256) = nk_set ? kf[KS + ks] : kf[ks];
        }
      }
      f32x4 s1 = {0.f, 0.f, 0.f, 0.f}, s2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s1 = mfma16x16x32<DT>(kf[ks], qf[ks], s1);
        s2 = mfma16x16x32<DT>(kf[KS + ks], qf[ks], s2);
      }
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_k(s + NW);
        asm volatile("" ::: "memory");
      }

      // Lane (head n16, q4) now holds scores of step tokens 8*q4 + i, i = 0..7.
      const int tb = 8 * q4;
      float sc[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[j] = (n16 < G && tb + j < nvalid) ? s1[j] * a.scale_log2 : -INFINITY;
        sc[4 + j] = (n16 < G && tb + 4 + j < nvalid) ? s2[j] * a.scale_log2 : -INFINITY;
      }
      float bmax = sc[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) bmax = fmaxf(bmax, sc[i]);
      bmax = group4_max(bmax);

      const bool need = (n16 < G) && (bmax > m_run + kLazyRescaleLog2);
      if (__any(need)) {
        const float m_new = need ? bmax : m_run;
        const float alpha = need ? fast_exp2(m_run - m_new) : 1.0f;
        l_run *= alpha;
        m_run = m_new;
        // O row r = 4*q4 + j belongs to head r % G (hi rows r < G, lo rows G <= r < 2G).
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float f = __shfl(alpha, (4 * q4 + j) % G);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) o[nb][j] *= f;
        }
      }

      float pv[8];
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        pv[i] = (n16 < G) ? fast_exp2(sc[i] - m_run) : 0.f;
        psum += pv[i];
      }
      l_run += psum;

      // hi = the weights rounded to 16 bits, lo = the rounding residuals rounded to 16 bits.
      u32x4 hi, lo;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        hi[wd] = pack2<DT>(pv[2 * wd], pv[2 * wd + 1]);
        lo[wd] = pack2<DT>(pv[2 * wd] - low_half<DT>(hi[wd]), pv[2 * wd + 1] - high_half<DT>(hi[wd]));
      }
      // Lo rows G..2G-1 take the lo parts of heads 0..G-1: a row shift by G inside each 16-lane
      // row (DPP row_shr), valid for the lanes that use it (n16 >= G).
      u32x4 pa;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        const uint32_t lo_src = static_cast<uint32_t>(
            __builtin_amdgcn_mov_dpp(static_cast<int>(lo[wd]), 0x110 + G, 0xF, 0xF, false));
        pa[wd] = (n16 < G) ? hi[wd] : ((n16 < 2 * G) ? lo_src : 0u);
      }

      if (new_step) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(nv[nb]));
        if (q4 == nv_q4) {
          const int e = ntt & 7;
          const uint32_t sh = (e & 1) * 16;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
            for (int wd = 0; wd < 4; ++wd) {
              if (wd == (e >> 1)) vf[nb][wd] = (vf[nb][wd] & ~(0xFFFFu << sh)) | (nv[nb] << sh);
            }
          }
        }
        // Likewise the half of the V tile that holds the new token's 8-token half (the lanes
        // q4 == nv_q4: 16 dimensions x 8 tokens per store, whole lines), before the tail past
        // the context is zeroed below.
        if (a.v_out != nullptr && q4 == nv_q4) {
          int64_t tA, tB;
          tiles(s, tA, tB);
          uint16_t* vp = static_cast<uint16_t*>(a.v_out) + (in_b ? tB : tA) + v_in_tile;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<u32x4*>(vp + nb * 16 * 8) = vf[nb];
        }
      }
      if (nvalid < 32) {
        // Tokens past the context are stale (possibly NaN): zero them in V, never multiply them.
        const int keep = min(8, max(0, nvalid - tb));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) vf[nb] = keep_first(vf[nb], keep);
      }
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) o[nb] = mfma16x16x32<DT>(pa, vf[nb], o[nb]);
      if (prefetch) {
        asm volatile("" ::: "memory");
        load_v(s + NW);
        asm volatile("" ::: "memory");
      }
    };

    load_k(st);
    load_v(st);
    for (; st + NW < cend; st += NW) step(st, true);
    step(st, false);
  }

  // Per-head sums over the four lane groups.
  l_run = group4_sum(l_run);
  // Fold each head's lo row (G + h) into its hi row (h): afterwards O row h = 4*q4 + j, h < G.
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (G >= 4) {
        o[nb][j] += __shfl_down(o[nb][j], 16 * (G / 4));
      } else if (j + G < 4) {
        o[nb][j] += o[nb][j + G];
      }
    }
  }

  float (&sO)[NW][G][D] = *reinterpret_cast<float (*)[NW][G][D]>(smem);
  float (&sM)[NW][G] = *reinterpret_cast<float (*)[NW][G]>(smem + NW * G * D);
  float (&sL)[NW][G] = *reinterpret_cast<float (*)[NW][G]>(smem + NW * G * D + NW * G);
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = 4 * q4 + j;
      if (r < G) sO[w][r][nb * 16 + n16] = o[nb][j];
    }
  }
  if (q4 == 0 && n16 < G) {
    sM[w][n16] = m_run;
    sL[w][n16] = l_run;
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < G * D; idx += NW * 64) {
    const int h = idx / D;
    const int d = idx % D;
    float M = sM[0][h];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sM[ww][h]);
    float acc = 0.f, lsum = 0.f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float f = fast_exp2(sM[ww][h] - M);  // waves without a step hold m = -inf -> 0
      acc += f * sO[ww][h][d];
      lsum += f * sL[ww][h];
    }
    emit<DT_OUT>(a, b, g * G + h, p, nparts, d, D, M, lsum, acc);
  }
}

}  // namespace
}  // namespace pkv
