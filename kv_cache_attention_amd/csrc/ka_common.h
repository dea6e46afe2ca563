// Shared device helpers of the gfx950 attention kernels: vector types, the
// f32 -> bf16 storage rounding, cache-layout index maps and wave reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ka {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kKeyBlock = 64;        // positions per K-cache block
constexpr float kLog2e = 1.4426950408889634f;

// ---------------------------------------------------------------- bf16 codec
// Round-to-nearest-even of an f32 bit pattern to its top 16 bits.  NaN keeps
// its top half with the quiet bit set, so it can never round into +-inf.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x0040u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// --------------------------------------------------------- cache layouts
// Element counts per 16-byte vector: 8 bf16 or 4 f32.
template <bool BF16> struct Elem;
template <> struct Elem<true> { typedef uint16_t T; static constexpr int E = 8; };
template <> struct Elem<false> { typedef float T; static constexpr int E = 4; };

// K: [B][Hkv][C/64][D/E][64][E].  Index of the 16-byte vector holding
// dims E*c .. E*c+E-1 of position j in the (b, g) cache slab.
__device__ __forceinline__ size_t k_vec_index(int j, int c, int D, int E) {
  return ((size_t)(j >> 6) * (D / E) + c) * 64 + (j & 63);
}
// V, f32: [B][Hkv][C/4][D][4].  Vector holding positions 4*(j/4) .. +3 of dim d.
__device__ __forceinline__ size_t vf32_vec_index(int j, int d, int D) {
  return (size_t)(j >> 2) * D + d;
}
// V, bf16: [B][Hkv][C/32][4][D][8].  In each 32-position block, group
// g = 2 s + h holds positions {16 s + 4 h + 0..3, 16 s + 8 + 4 h + 0..3}
// (slots 0..3 and 4..7) -- the positions one lane half holds in the
// accumulator of a 32x32 MFMA, so exponentiated scores feed the value
// product directly.  For r = j % 32: g = 2 (r / 16) + (r % 8) / 4,
// t = r % 4 + 4 ((r % 16) / 8).
__device__ __forceinline__ int vbf16_group(int j) {
  return ((j >> 5) << 2) + (((j >> 4) & 1) << 1) + ((j >> 2) & 1);
}
__device__ __forceinline__ int vbf16_slot(int j) { return (j & 3) + (((j >> 3) & 1) << 2); }
// inverse: position of slot t in group g of 32-block blk
__device__ __forceinline__ int vbf16_pos(int blk, int g, int t) {
  return (blk << 5) + ((g >> 1) << 4) + ((g & 1) << 2) + (t & 3) + ((t >> 2) << 3);
}

// ------------------------------------------------------- wave reductions
// Butterfly max / sum across the 64 lanes of a wavefront (every lane ends
// with the result).  NaN reaching these is handled by the callers.
__device__ __forceinline__ float xor_shfl(float x, int m) { return __shfl_xor(x, m, kWave); }

template <int WIDTH>
__device__ __forceinline__ float group_max(float x) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) x = fmaxf(x, xor_shfl(x, m));
  return x;
}
template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
#pragma unroll
  for (int m = 1; m < WIDTH; m <<= 1) x += xor_shfl(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace ka
