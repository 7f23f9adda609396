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
