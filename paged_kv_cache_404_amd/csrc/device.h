// Device-side types and small helpers shared by the HIP kernels of libpagedkv (gfx950 / CDNA4).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pagedkv.h"
#include "status.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kBlock = 16;  // tokens per physical block (the kernels' only block size)

inline hipStream_t as_stream(pkv_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

inline int elem_size(int32_t dtype) { return dtype == PKV_F32 ? 4 : 2; }

inline bool valid_dtype(int32_t dtype) { return dtype == PKV_F32 || dtype == PKV_F16 || dtype == PKV_BF16; }

// Returns PKV_EHIP with the launch error, or PKV_OK.
inline int check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(PKV_EHIP, "%s: kernel launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

// 16-bit element <-> float.
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __builtin_bit_cast(float, bits16 << 16);
}
__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits16)));
}

// Copy one element of type DT, bit for bit: dst[di] = src[si].
template <int DT>
__device__ __forceinline__ void copy_elem(void* dst, int64_t di, const void* src, int64_t si) {
  if constexpr (DT == PKV_F32) {
    static_cast<uint32_t*>(dst)[di] = static_cast<const uint32_t*>(src)[si];
  } else {
    static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
  }
}

template <int DT>
__device__ __forceinline__ float elem_to_float(const void* base, int64_t i) {
  if constexpr (DT == PKV_F32) {
    return static_cast<const float*>(base)[i];
  } else if constexpr (DT == PKV_BF16) {
    return bf16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
  } else {
    return f16_bits_to_float(static_cast<const uint16_t*>(base)[i]);
  }
}

template <int DT>
__device__ __forceinline__ void store_from_float(void* base, int64_t i, float x) {
  if constexpr (DT == PKV_F32) {
    static_cast<float*>(base)[i] = x;
  } else if constexpr (DT == PKV_BF16) {
    static_cast<__bf16*>(base)[i] = static_cast<__bf16>(x);  // round to nearest even
  } else {
    static_cast<_Float16*>(base)[i] = static_cast<_Float16>(x);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

constexpr float kLog2e = 1.4426950408889634f;
// Lazy rescale threshold (log2 domain): the running maximum moves only when a score exceeds it
// by more than 2^8, so softmax weights stay <= 256 and rescaling is rare.
constexpr float kLazyRescaleLog2 = 8.0f;

// One v_mfma_f32_16x16x32_{bf16,f16}: C += A (16x32) . B (32x16), fragments of 8 16-bit elements.
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

// Two floats -> two 16-bit elements of the matrix-core input type in one 32-bit word (low half =
// a), round to nearest even: one v_cvt_pk_{bf16,f16}_f32.
template <int DT>
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  const f32x2 x = {a, b};
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
}
// The low / high 16-bit element of a packed word, widened exactly to float.
template <int DT>
__device__ __forceinline__ float low_half(uint32_t w) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(float, w << 16);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w)));
  }
}
template <int DT>
__device__ __forceinline__ float high_half(uint32_t w) {
  if constexpr (DT == PKV_BF16) {
    return __builtin_bit_cast(float, w & 0xFFFF0000u);
  } else {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(w >> 16)));
  }
}

// Reductions over the four 16-lane groups of a wave (lanes n, n + 16, n + 32, n + 48), every
// lane receiving the result.  gfx950's v_permlane16_swap / v_permlane32_swap exchange 16-lane
// rows (lane i <-> i ^ 16) and 32-lane halves (i <-> i ^ 32) inside the VALU, instead of a
// round trip through the LDS crossbar (ds_bpermute).  Each step combines the same two values
// in the same order as x op shfl_xor(x, 16 or 32), so results are bit-identical to that form.
__device__ __forceinline__ float swap16_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float group4_max(float x) { return swap32_max(swap16_max(x)); }
__device__ __forceinline__ float group4_sum(float x) { return swap32_sum(swap16_sum(x)); }

// K tile order.  A (block, head) K tile holds 16 tokens x head_dim elements as 16-byte chunks;
// chunk c of token t (elements [c*E, c*E + E) of that token's head vector, E = 16 / elem_size)
// sits at chunk index
//     ((c / 4) * 2 + (t / 4) % 2) * 32 + (c % 4) * 8 + (t / 8) * 4 + t % 4
// i.e. the tile is [c / 4][token set (t / 4) % 2][c % 4][8 tokens of the set].  One matrix-core
// k-step of a 32-token step (two blocks) then reads one 512-byte run from each block: every
// cache line is fully used by a single load instruction.
__host__ __device__ __forceinline__ int k_chunk_pos(int t, int c) {
  return ((c >> 2) * 2 + ((t >> 2) & 1)) * 32 + (c & 3) * 8 + (t >> 3) * 4 + (t & 3);
}

}  // namespace pkv
