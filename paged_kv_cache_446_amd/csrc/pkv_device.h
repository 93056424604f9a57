// Device-side building blocks shared by the gfx950 kernels of libpkv.
//
// Tile layouts (see include/pkv.h): a K tile is [D/x][16][x] and a V tile is
// [D/(16*x4)][4][16][x4][4] with x = 16 / element bytes, x4 = x / 4.  Read as
// 16-byte chunks, chunk (m * 64 + lane) of either tile is exactly what lane
// `lane` of a 64-wide wavefront needs as a matrix-instruction operand:
//
//   K chunk kk*64 + lane, lane = 16*g + c:  K[token c][dims (kk*4+g)*x .. +x)
//       -> A operand of S^T = K . Q^T  (rows = tokens, k = head dims)
//   V chunk m*64 + lane:  V[tokens 4g .. 4g+3][dim (m*x4 + r)*16 + c], r < x4
//       -> A operand of O^T = V^T . P^T (rows = head dims, k = tokens)
//
// and the S^T result (lane 16g+c holds tokens 4g..4g+3 of column c) is
// already the B operand layout of the P^T side.  No LDS transpose is needed.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;

constexpr int kBlock = 16;  // tokens per KV block
constexpr int kWave = 64;

typedef uint32_t u32v4 __attribute__((ext_vector_type(4)));  // the same 16 bytes as a vector
struct alignas(16) u32x4 {
  uint32_t x, y, z, w;
};

// ---- element types --------------------------------------------------------

struct TF32 {
  typedef float T;
  static constexpr int kBytes = 4;
};
struct TF16 {
  typedef _Float16 T;
  static constexpr int kBytes = 2;
};
struct TBF16 {
  typedef uint16_t T;  // raw bits; converted by hand
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 -> bf16, round to nearest even: gfx950 converts in hardware (v_cvt_pk_bf16_f32)
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// pack two fp32 values as 2 x 16-bit elements into one dword
__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  const bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ uint32_t pack2_f16(float a, float b) {
  _Float16 ha = (_Float16)a, hb = (_Float16)b;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, ha) | ((uint32_t)__builtin_bit_cast(uint16_t, hb) << 16);
}

// ---- matrix instructions ---------------------------------------------------

// S^T += K . Q^T over 32 head dims (16-bit types): a = 8 K elems, b = 8 Q elems
__device__ __forceinline__ f32x4 mma_k32(const u32x4& a, const u32x4& b, f32x4 c, TBF16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k32(const u32x4& a, const u32x4& b, f32x4 c, TF16) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// 16 x 16 x 16 with 4 elements per lane (16-bit types): a, b = 2 dwords each
__device__ __forceinline__ f32x4 mma_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                         f32x4 c, TBF16) {
  uint2 a = make_uint2(a0, a1), b = make_uint2(b0, b1);
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                   __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma_k16(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1,
                                         f32x4 c, TF16) {
  uint2 a = make_uint2(a0, a1), b = make_uint2(b0, b1);
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                               __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
}

// 16 x 16 x 4, fp32: one element per lane
__device__ __forceinline__ f32x4 mma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ---- cross-lane ------------------------------------------------------------

__device__ __forceinline__ float shfl_xor(float v, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(v)));
}

__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pkv
