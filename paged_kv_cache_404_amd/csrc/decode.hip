// Paged decode attention: block-table gather, scaled Q.K, online softmax, P.V, GQA groups, and a
// split-K partition + log-sum-exp reduce for long contexts.
//
// What is computed ([Serving] "Production Serving: Continuous Batching and PagedAttention", The
// Build, Step 6): for each sequence b and query head h, every cached token t < L_b is scored
// s_t = scale * <q_{b,h}, K_{g,t}> against KV head g = h / (Hq / Hkv); the scores are
// softmaxed and the output is sum_t w_t V_{g,t}.  Tokens are found through the block table;
// the unused tail of the last block is skipped, never multiplied by zero (stale slots may hold
// NaN).
//
// Split-K: the context is cut into fixed partitions of `part_size` tokens (boundaries depend on
// the position only).  Each partition keeps the usual online-softmax state (reference maximum m,
// sum l, unnormalised output o); partitions of one (sequence, head) are merged exactly:
// M = max_p m_p, out = sum_p 2^(m_p - M) o_p / sum_p 2^(m_p - M) l_p.
//
// MI355X mapping (bf16 / fp16): one wavefront handles 32 tokens (two 16-token blocks) of one KV
// head per step.  The GQA group's query rows share every K/V tile load.  Both products run on the
// matrix cores with v_mfma_f32_16x16x32_{bf16,f16}:
//   S^T[token][head] = K[token][:] . Q[head][:]      (A = K rows, B = Q^T, heads padded to 16)
//   O[row][d]       += P[row][token] . V[token][d]    (A = P rows, B = V^T tile)
// The V cache is stored dim-major per block ([D][16]) so that eight consecutive tokens of one
// dimension are one 16-byte load, which is what the P.V operand wants.  The softmax weights are
// fed as two 16-bit rows, hi = round(p) and lo = round(p - hi), in the padding rows of the same
// MFMA, so P.V keeps ~16 mantissa bits at no extra matrix instruction.  Scores use exp2 with
// log2(e) folded into the scale; the running maximum is only raised when a score exceeds it by
// more than 2^8 (lazy rescaling: exact, and p stays <= 256), which makes rescaling rare.
#include <algorithm>
#include <cmath>
#include <type_traits>

#include "device.h"

namespace pkv {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyRescaleLog2 = 8.0f;

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
  int32_t num_order;  // 0, or B: workgroup row y works on sequence order[y]
  int32_t order[kMaxOrder];
};

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

template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0,
                                                  0, 0);
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
template <int DT, int DT_OUT, int D, int G, int NW, bool NEWTOK>
__global__ void __launch_bounds__(NW * 64) decode_mfma_kernel(DecodeArgs a) {
  static_assert(D == 64 || D == 128, "head_dim");
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  constexpr int KS = D / 32;        // k-steps of Q.K
  constexpr int NB = D / 16;        // 16-column blocks of P.V
  constexpr int TILE = kBlock * D;  // elements of one (block, head) tile
  constexpr int kTableSteps = 32;   // steps covered by one block-id load (64 blocks, one per lane)

  const int g = blockIdx.x;
  const int b = a.num_order ? a.order[blockIdx.y] : static_cast<int>(blockIdx.y);
  const int p = blockIdx.z;
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
  // (8 consecutive tokens of one dimension) is one 16-byte load from the dim-major V tile.
  const int k_in_tile = (q4 * 8 + (n16 & 7)) * 8;  // chunk (k-step 0, set 0) of this lane, in elements
  const bool k_from_b = n16 >= 8;
  const bool v_from_b = q4 >= 2;
  const int v_in_tile = n16 * kBlock + (q4 & 1) * 8;

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
        vf[nb] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vp + nb * 16 * kBlock));
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
        // The registers now hold the new token's whole K tile (the other slots as loaded):
        // store it back with the load's own lane pattern, so every cache line is written whole.
        // Without k_out the caller writes the cache itself (paged_attention_decode_newest).
        if (a.k_out != nullptr && k_from_b == in_b) {
          int64_t tA, tB;
          tiles(s, tA, tB);
          uint16_t* kp = static_cast<uint16_t*>(a.k_out) + (in_b ? tB : tA) + k_in_tile;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            *reinterpret_cast<u32x4*>(kp + (2 * ks) * 256) = kf[ks];
            *reinterpret_cast<u32x4*>(kp + (2 * ks + 1) * 256) = kf[KS + ks];
          }
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
        // Likewise the whole V tile, before the tail past the context is zeroed below.
        if (a.v_out != nullptr && v_from_b == in_b) {
          int64_t tA, tB;
          tiles(s, tA, tB);
          uint16_t* vp = static_cast<uint16_t*>(a.v_out) + (in_b ? tB : tA) + v_in_tile;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) *reinterpret_cast<u32x4*>(vp + nb * 16 * kBlock) = vf[nb];
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

  __shared__ float sO[NW][G][D];
  __shared__ float sM[NW][G];
  __shared__ float sL[NW][G];
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

// ------------------------------------------------------------------------------------------
// Vector-ALU kernel (any element type; used for fp32).  grid = (Hq, B, max_parts), one wave.
// Lane i scores token c0 + i of each 64-token chunk; each lane owns dims lane and lane + 64.
// ------------------------------------------------------------------------------------------
template <int DT, int DT_OUT, int D>
__global__ void __launch_bounds__(64) decode_valu_kernel(DecodeArgs a) {
  constexpr int E = DT == PKV_F32 ? 4 : 8;  // elements per 16-byte chunk of the K tile
  const int hq = blockIdx.x;
  const int b = a.num_order ? a.order[blockIdx.y] : static_cast<int>(blockIdx.y);
  const int p = blockIdx.z;
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

  constexpr int DPL = (D + 63) / 64;  // dims per lane
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  for (int c0 = pstart; c0 < pend; c0 += 64) {
    const int t = c0 + lane;
    const bool valid = t < pend;
    int64_t tile = 0;
    int off = 0;
    float s = -INFINITY;
    if (valid) {
      tile = (static_cast<int64_t>(clamp_blk(a, table[t / kBlock])) * a.Hkv + g) * kBlock * D;
      off = t % kBlock;
      float acc = 0.f;
      for (int d = 0; d < D; ++d)
        acc += qs[d] * elem_to_float<DT>(a.k, tile + static_cast<int64_t>(k_chunk_pos(off, d / E)) * E + d % E);
      s = acc;
    }
    const float m_new = fmaxf(m_run, wave_max(s));
    const float alpha = fast_exp2(m_run - m_new);
    const float pt = valid ? fast_exp2(s - m_new) : 0.f;
    l_run = l_run * alpha + wave_sum(pt);
#pragma unroll
    for (int i = 0; i < DPL; ++i) o[i] *= alpha;
    const int n = min(64, pend - c0);
    for (int i = 0; i < n; ++i) {
      const float pi = __shfl(pt, i);
      const int64_t ti = __shfl(tile, i);
      const int oi = __shfl(off, i);
#pragma unroll
      for (int k = 0; k < DPL; ++k) {
        const int d = lane + 64 * k;
        if (d < D) o[k] += pi * elem_to_float<DT>(a.v, ti + static_cast<int64_t>(d) * kBlock + oi);
      }
    }
    m_run = m_new;
  }
#pragma unroll
  for (int k = 0; k < DPL; ++k) {
    const int d = lane + 64 * k;
    if (d < D) emit<DT_OUT>(a, b, hq, p, nparts, d, D, m_run, l_run, o[k]);
  }
}

// ------------------------------------------------------------------------------------------
// Log-sum-exp merge of partitions.  grid = (Hq, B), 128 threads.  MAXP >= max_parts (up to 64):
// every partial of the row is loaded at once, together with the context length (one memory
// latency), (m, l) through LDS; the sequence's own partition count then selects which take
// part.  Rows of single-partition sequences were written by the partition pass and are left
// alone.
// ------------------------------------------------------------------------------------------
template <int DT_OUT, int MAXP>
__global__ void __launch_bounds__(128) decode_reduce_kernel(void* __restrict__ out, const float* __restrict__ part_ml,
                                                            const float* __restrict__ part_o,
                                                            const int32_t* __restrict__ lens, int32_t Hq, int32_t D,
                                                            int32_t max_parts, int32_t part_size) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int64_t row0 = (static_cast<int64_t>(b) * Hq + h) * max_parts;
  __shared__ float sm[MAXP], sl[MAXP];
  // Thread p fetches partition p's (m, l); every thread fetches its dimension of every partial.
  if (d < MAXP) {
    const bool in = d < max_parts;
    sm[d] = in ? part_ml[(row0 + d) * 2] : -INFINITY;
    sl[d] = in ? part_ml[(row0 + d) * 2 + 1] : 0.f;
  }
  float o[MAXP];
#pragma unroll
  for (int p = 0; p < MAXP; ++p) o[p] = (p < max_parts && d < D) ? part_o[(row0 + p) * D + d] : 0.f;
  const int L = min(lens[b], max_parts * part_size);
  const int nparts = (L + part_size - 1) / part_size;
  __syncthreads();
  if (nparts <= 1 || d >= D) return;
  float M = -INFINITY;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) M = p < nparts ? fmaxf(M, sm[p]) : M;
  float acc = 0.f, lsum = 0.f;
#pragma unroll
  for (int p = 0; p < MAXP; ++p) {
    if (p < nparts) {
      const float f = fast_exp2(sm[p] - M);
      acc += f * o[p];
      lsum += f * sl[p];
    }
  }
  store_from_float<DT_OUT>(out, (static_cast<int64_t>(b) * Hq + h) * D + d, acc / lsum);
}

// Any number of partitions: the same merge, loads in a loop.
template <int DT_OUT>
__global__ void __launch_bounds__(128) decode_reduce_loop_kernel(void* __restrict__ out,
                                                                 const float* __restrict__ part_ml,
                                                                 const float* __restrict__ part_o,
                                                                 const int32_t* __restrict__ lens, int32_t Hq,
                                                                 int32_t D, int32_t max_parts, int32_t part_size) {
  const int h = blockIdx.x;
  const int b = blockIdx.y;
  const int d = threadIdx.x;
  const int L = min(lens[b], max_parts * part_size);
  const int nparts = (L + part_size - 1) / part_size;
  if (nparts <= 1 || d >= D) return;
  const int64_t row0 = (static_cast<int64_t>(b) * Hq + h) * max_parts;
  const float* ml = part_ml + row0 * 2;
  float M = -INFINITY;
  for (int p = 0; p < nparts; ++p) M = fmaxf(M, ml[2 * p]);
  float acc = 0.f, lsum = 0.f;
  for (int p = 0; p < nparts; ++p) {
    const float f = fast_exp2(ml[2 * p] - M);
    acc += f * part_o[(row0 + p) * D + d];
    lsum += f * ml[2 * p + 1];
  }
  store_from_float<DT_OUT>(out, (static_cast<int64_t>(b) * Hq + h) * D + d, acc / lsum);
}

// ------------------------------------------------------------------------------------------
// Host side
// ------------------------------------------------------------------------------------------
struct Plan {
  int32_t part_size;
  int32_t max_parts;
  size_t ml_bytes;
  size_t need_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

Plan make_plan(int32_t B, int32_t Hq, int32_t D, int32_t max_ctx, int32_t partition_size) {
  Plan pl{};
  if (partition_size <= 0) {
    pl.part_size = ((max_ctx + kBlock - 1) / kBlock) * kBlock;
    if (pl.part_size < kBlock) pl.part_size = kBlock;
    pl.max_parts = 1;
    pl.ml_bytes = 0;
    pl.need_bytes = 0;
  } else {
    pl.part_size = partition_size;
    pl.max_parts = (max_ctx + partition_size - 1) / partition_size;
    pl.ml_bytes = align256(static_cast<size_t>(B) * Hq * pl.max_parts * 2 * sizeof(float));
    pl.need_bytes = pl.ml_bytes + static_cast<size_t>(B) * Hq * pl.max_parts * D * sizeof(float);
  }
  return pl;
}

int validate(const char* fn, void* out, int32_t out_dtype, const void* query, const void* k_cache,
             const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t Hq,
             int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks, int32_t num_blocks, int32_t max_ctx,
             int32_t partition_size, const void* workspace, size_t workspace_bytes, int32_t dtype) {
  if (!valid_dtype(dtype)) return fail(PKV_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (out_dtype != PKV_F32 && out_dtype != dtype)
    return fail(PKV_EINVAL, "%s: out_dtype must be PKV_F32 or the input dtype", fn);
  if (B < 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || bs <= 0 || max_blocks < 0 || num_blocks <= 0 || max_ctx < 0)
    return fail(PKV_EINVAL, "%s: bad sizes", fn);
  if (Hq % Hkv != 0) return fail(PKV_EINVAL, "%s: num_q_heads %d not a multiple of num_kv_heads %d", fn, Hq, Hkv);
  if (bs != kBlock) return fail(PKV_EUNSUPPORTED, "%s: block_size %d (kernels implement 16)", fn, bs);
  if (D != 64 && D != 128) return fail(PKV_EUNSUPPORTED, "%s: head_dim %d (64 or 128)", fn, D);
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8) return fail(PKV_EUNSUPPORTED, "%s: group size %d", fn, G);
  if (B > 65535 || Hq > 65535) return fail(PKV_EUNSUPPORTED, "%s: batch or head count above 65535", fn);
  if (partition_size != PKV_SINGLE_PASS_ADAPTIVE && (partition_size < 0 || partition_size % bs != 0))
    return fail(PKV_EINVAL, "%s: partition_size %d must be 0, -1 or a multiple of block_size", fn, partition_size);
  if (partition_size > 0 && (max_ctx + static_cast<int64_t>(partition_size) - 1) / partition_size > 65535)
    return fail(PKV_EUNSUPPORTED, "%s: more than 65535 partitions per sequence", fn);
  if (static_cast<int64_t>(max_ctx) > static_cast<int64_t>(max_blocks) * bs)
    return fail(PKV_EINVAL, "%s: max_context_len %d exceeds max_blocks_per_seq * block_size", fn, max_ctx);
  if (B == 0) return PKV_OK;
  if (!out || !query || !k_cache || !v_cache || !block_tables || !context_lens)
    return fail(PKV_EINVAL, "%s: NULL pointer", fn);
  const Plan pl = make_plan(B, Hq, D, max_ctx, partition_size);
  if (pl.need_bytes > 0 && (!workspace || workspace_bytes < pl.need_bytes))
    return fail(PKV_EINVAL, "%s: workspace of %zu bytes needed, %zu given", fn, pl.need_bytes, workspace_bytes);
  const uintptr_t al = reinterpret_cast<uintptr_t>(query) | reinterpret_cast<uintptr_t>(k_cache) |
                       reinterpret_cast<uintptr_t>(v_cache) | reinterpret_cast<uintptr_t>(workspace);
  if (al % 16 != 0) return fail(PKV_EINVAL, "%s: query, caches and workspace must be 16-byte aligned", fn);
  return PKV_OK;
}

template <int DT, int DT_OUT, int D>
int launch_valu(const DecodeArgs& a, int B, hipStream_t s) {
  hipLaunchKernelGGL((decode_valu_kernel<DT, DT_OUT, D>), dim3(a.Hq, B, a.max_parts), dim3(64), 0, s, a);
  return PKV_OK;
}

// Waves per workgroup: 4 for partitions of up to 512 tokens (<= 4 steps per wave), 8 above and
// for the single pass.  The choice depends only on the caller's partition_size, never on the
// batch (a single pass spans the batch's longest context, so its wave count is fixed): a
// sequence's reduction order, and so its output bits, do not depend on the rest of the batch.
// The batch-adaptive single pass (partition_size -1) applies the 512-token rule to the batch's
// longest context instead.
template <int DT, int DT_OUT, int D, int G>
int launch_mfma(const DecodeArgs& a, int B, bool single_pass, hipStream_t s) {
  const dim3 grid(a.Hkv, B, a.max_parts);
  const bool fused = a.new_k != nullptr;
  if (!single_pass && a.part_size <= 512) {
    if (fused)
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 4, true>), grid, dim3(256), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 4, false>), grid, dim3(256), 0, s, a);
  } else {
    if (fused)
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 8, true>), grid, dim3(512), 0, s, a);
    else
      hipLaunchKernelGGL((decode_mfma_kernel<DT, DT_OUT, D, G, 8, false>), grid, dim3(512), 0, s, a);
  }
  return PKV_OK;
}

template <int DT, int DT_OUT, int D>
int dispatch_group(const DecodeArgs& a, int B, bool single_pass, hipStream_t s) {
  switch (a.Hq / a.Hkv) {
    case 1: return launch_mfma<DT, DT_OUT, D, 1>(a, B, single_pass, s);
    case 2: return launch_mfma<DT, DT_OUT, D, 2>(a, B, single_pass, s);
    case 4: return launch_mfma<DT, DT_OUT, D, 4>(a, B, single_pass, s);
    default: return launch_mfma<DT, DT_OUT, D, 8>(a, B, single_pass, s);
  }
}

template <int DT, int DT_OUT>
int dispatch_dim(const DecodeArgs& a, int D, int B, bool single_pass, hipStream_t s) {
  if constexpr (DT == PKV_F32) {
    return D == 64 ? launch_valu<DT, DT_OUT, 64>(a, B, s) : launch_valu<DT, DT_OUT, 128>(a, B, s);
  } else {
    return D == 64 ? dispatch_group<DT, DT_OUT, 64>(a, B, single_pass, s)
                   : dispatch_group<DT, DT_OUT, 128>(a, B, single_pass, s);
  }
}

int launch_partitions(const DecodeArgs& a, int32_t dtype, int32_t out_dtype, int D, int B, bool single_pass,
                      hipStream_t s) {
  const bool f32out = out_dtype == PKV_F32;
  switch (dtype) {
    case PKV_BF16:
      return f32out ? dispatch_dim<PKV_BF16, PKV_F32>(a, D, B, single_pass, s)
                    : dispatch_dim<PKV_BF16, PKV_BF16>(a, D, B, single_pass, s);
    case PKV_F16:
      return f32out ? dispatch_dim<PKV_F16, PKV_F32>(a, D, B, single_pass, s)
                    : dispatch_dim<PKV_F16, PKV_F16>(a, D, B, single_pass, s);
    default:
      return dispatch_dim<PKV_F32, PKV_F32>(a, D, B, single_pass, s);
  }
}

template <int DT_OUT>
void launch_reduce_t(void* out, const float* ml, const float* po, const int32_t* lens, int B, int Hq, int D,
                     int max_parts, int part_size, hipStream_t s) {
  const dim3 grid(Hq, B), block(128);
  if (max_parts <= 4)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 4>), grid, block, 0, s, out, ml, po, lens, Hq, D, max_parts,
                       part_size);
  else if (max_parts <= 8)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 8>), grid, block, 0, s, out, ml, po, lens, Hq, D, max_parts,
                       part_size);
  else if (max_parts <= 16)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 16>), grid, block, 0, s, out, ml, po, lens, Hq, D, max_parts,
                       part_size);
  else if (max_parts <= 32)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 32>), grid, block, 0, s, out, ml, po, lens, Hq, D, max_parts,
                       part_size);
  else if (max_parts <= 64)
    hipLaunchKernelGGL((decode_reduce_kernel<DT_OUT, 64>), grid, block, 0, s, out, ml, po, lens, Hq, D, max_parts,
                       part_size);
  else
    hipLaunchKernelGGL((decode_reduce_loop_kernel<DT_OUT>), grid, dim3(D), 0, s, out, ml, po, lens, Hq, D,
                       max_parts, part_size);
}

int launch_reduce(void* out, int32_t out_dtype, const float* ml, const float* po, const int32_t* lens, int B, int Hq,
                  int D, int max_parts, int part_size, hipStream_t s) {
  switch (out_dtype) {
    case PKV_BF16: launch_reduce_t<PKV_BF16>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
    case PKV_F16: launch_reduce_t<PKV_F16>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
    default: launch_reduce_t<PKV_F32>(out, ml, po, lens, B, Hq, D, max_parts, part_size, s); break;
  }
  return PKV_OK;
}

}  // namespace
}  // namespace pkv

using namespace pkv;

extern "C" size_t paged_attention_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim,
                                                         int32_t max_context_len, int32_t partition_size) {
  if (num_seqs <= 0 || num_q_heads <= 0 || head_dim <= 0 || max_context_len <= 0 || partition_size <= 0) return 0;
  return make_plan(num_seqs, num_q_heads, head_dim, max_context_len, partition_size).need_bytes;
}

namespace pkv {
namespace {

// Partition pass shared by the plain and the fused-append entry points (new_k == nullptr: plain).
int partitions_impl(const char* fn, void* out, int32_t out_dtype, const void* query, const void* k_cache,
                    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                    int32_t Hq, int32_t Hkv, int32_t D, int32_t bs, int32_t max_blocks, int32_t num_blocks,
                    int32_t max_ctx, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
                    int32_t dtype, const void* new_k, const void* new_v, void* k_out, void* v_out,
                    const int32_t* host_lens, pkv_stream_t stream) {
  int st = validate(fn, out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B, Hq, Hkv, D, bs,
                    max_blocks, num_blocks, max_ctx, partition_size, workspace, workspace_bytes, dtype);
  if (st != PKV_OK || B == 0 || max_ctx == 0) return st;
  if (new_k != nullptr || new_v != nullptr) {
    if (dtype == PKV_F32) return fail(PKV_EUNSUPPORTED, "%s: fused append needs bf16 or fp16 caches", fn);
    if (!new_k || !new_v) return fail(PKV_EINVAL, "%s: NULL new_key or new_value", fn);
    if ((reinterpret_cast<uintptr_t>(new_k) | reinterpret_cast<uintptr_t>(new_v)) % 16 != 0)
      return fail(PKV_EINVAL, "%s: new_key and new_value must be 16-byte aligned", fn);
  }
  const Plan pl = make_plan(B, Hq, D, max_ctx, partition_size);
  DecodeArgs a{};
  a.out = out;
  a.q = query;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.lens = context_lens;
  a.part_ml = pl.need_bytes ? static_cast<float*>(workspace) : nullptr;
  a.part_o = pl.need_bytes ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + pl.ml_bytes) : nullptr;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.max_blocks = max_blocks;
  a.num_blocks = num_blocks;
  a.max_parts = pl.max_parts;
  a.part_size = pl.part_size;
  a.scale_log2 = scale * kLog2e;
  a.new_k = new_k;
  a.new_v = new_v;
  a.k_out = k_out;
  a.v_out = v_out;
  if (host_lens != nullptr && B <= kMaxOrder) {
    // Longest sequences first (ties by index): the scheduling order only, never the arithmetic.
    for (int i = 0; i < B; ++i) a.order[i] = i;
    std::stable_sort(a.order, a.order + B, [&](int32_t x, int32_t y) { return host_lens[x] > host_lens[y]; });
    a.num_order = B;
  }
  launch_partitions(a, dtype, out_dtype, D, B, partition_size == 0, as_stream(stream));
  return check_launch(fn);
}

}  // namespace
}  // namespace pkv

extern "C" int paged_attention_decode_partitions(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                                 const void* v_cache, const int32_t* block_tables,
                                                 const int32_t* context_lens, int32_t B, int32_t num_q_heads,
                                                 int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                                 int32_t max_blocks_per_seq, int32_t num_blocks,
                                                 int32_t max_context_len, float scale, int32_t partition_size,
                                                 void* workspace, size_t workspace_bytes, int32_t dtype,
                                                 const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_partitions", out, out_dtype, query, k_cache, v_cache, block_tables,
                         context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                         num_blocks, max_context_len, scale, partition_size, workspace, workspace_bytes, dtype,
                         nullptr, nullptr, nullptr, nullptr, host_context_lens, stream);
}

extern "C" int paged_attention_decode_append_partitions(
    void* out, int32_t out_dtype, const void* query, const void* new_key, const void* new_value, void* k_cache,
    void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_append_partitions", out, out_dtype, query, k_cache, v_cache,
                         block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                         workspace_bytes, dtype, new_key, new_value, k_cache, v_cache, host_context_lens, stream);
}

extern "C" int paged_attention_decode_reduce(void* out, int32_t out_dtype, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t head_dim, int32_t max_context_len,
                                             int32_t partition_size, const void* workspace, size_t workspace_bytes,
                                             pkv_stream_t stream) {
  if (B < 0 || num_q_heads <= 0 || (head_dim != 64 && head_dim != 128) || max_context_len < 0 ||
      partition_size < PKV_SINGLE_PASS_ADAPTIVE)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: bad sizes");
  if (out_dtype != PKV_F32 && out_dtype != PKV_F16 && out_dtype != PKV_BF16)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: unknown out_dtype %d", out_dtype);
  if (partition_size > 0 && partition_size % kBlock != 0)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: partition_size must be a multiple of 16");
  if (B == 0 || max_context_len == 0 || partition_size <= 0) return PKV_OK;
  const Plan pl = make_plan(B, num_q_heads, head_dim, max_context_len, partition_size);
  if (pl.max_parts <= 1) return PKV_OK;
  if (!out || !context_lens || !workspace || workspace_bytes < pl.need_bytes)
    return fail(PKV_EINVAL, "paged_attention_decode_reduce: NULL pointer or workspace too small");
  const float* ml = static_cast<const float*>(workspace);
  const float* po = reinterpret_cast<const float*>(static_cast<const uint8_t*>(workspace) + pl.ml_bytes);
  launch_reduce(out, out_dtype, ml, po, context_lens, B, num_q_heads, head_dim, pl.max_parts, pl.part_size,
                as_stream(stream));
  return check_launch("paged_attention_decode_reduce");
}

extern "C" int paged_attention_decode(void* out, int32_t out_dtype, const void* query, const void* k_cache,
                                      const void* v_cache, const int32_t* block_tables, const int32_t* context_lens,
                                      int32_t B, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                      int32_t max_context_len, float scale, int32_t partition_size, void* workspace,
                                      size_t workspace_bytes, int32_t dtype, const int32_t* host_context_lens,
                                      pkv_stream_t stream) {
  int st = paged_attention_decode_partitions(out, out_dtype, query, k_cache, v_cache, block_tables, context_lens, B,
                                             num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                                             num_blocks, max_context_len, scale, partition_size, workspace,
                                             workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_append(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, void* k_cache, void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = paged_attention_decode_append_partitions(out, out_dtype, query, new_key, new_value, k_cache, v_cache,
                                                    block_tables, context_lens, B, num_q_heads, num_kv_heads,
                                                    head_dim, block_size, max_blocks_per_seq, num_blocks,
                                                    max_context_len, scale, partition_size, workspace,
                                                    workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}

extern "C" int paged_attention_decode_newest_partitions(
    void* out, int32_t out_dtype, const void* query, const void* new_key, const void* new_value, const void* k_cache,
    const void* v_cache, const int32_t* block_tables, const int32_t* context_lens, int32_t B, int32_t num_q_heads,
    int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
    int32_t max_context_len, float scale, int32_t partition_size, void* workspace, size_t workspace_bytes,
    int32_t dtype, const int32_t* host_context_lens, pkv_stream_t stream) {
  return partitions_impl("paged_attention_decode_newest_partitions", out, out_dtype, query, k_cache, v_cache,
                         block_tables, context_lens, B, num_q_heads, num_kv_heads, head_dim, block_size,
                         max_blocks_per_seq, num_blocks, max_context_len, scale, partition_size, workspace,
                         workspace_bytes, dtype, new_key, new_value, nullptr, nullptr, host_context_lens, stream);
}

extern "C" int paged_attention_decode_newest(void* out, int32_t out_dtype, const void* query, const void* new_key,
                                             const void* new_value, const void* k_cache, const void* v_cache,
                                             const int32_t* block_tables, const int32_t* context_lens, int32_t B,
                                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                             int32_t block_size, int32_t max_blocks_per_seq, int32_t num_blocks,
                                             int32_t max_context_len, float scale, int32_t partition_size,
                                             void* workspace, size_t workspace_bytes, int32_t dtype,
                                             const int32_t* host_context_lens, pkv_stream_t stream) {
  int st = paged_attention_decode_newest_partitions(out, out_dtype, query, new_key, new_value, k_cache, v_cache,
                                                    block_tables, context_lens, B, num_q_heads, num_kv_heads,
                                                    head_dim, block_size, max_blocks_per_seq, num_blocks,
                                                    max_context_len, scale, partition_size, workspace,
                                                    workspace_bytes, dtype, host_context_lens, stream);
  if (st != PKV_OK) return st;
  return paged_attention_decode_reduce(out, out_dtype, context_lens, B, num_q_heads, head_dim, max_context_len,
                                       partition_size, workspace, workspace_bytes, stream);
}
