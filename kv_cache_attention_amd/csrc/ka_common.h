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
// Cache element formats: kv_dtype 0 = f32, 1 = bf16, 2 = int8 K codes (with
// one f32 scale per row) and bf16 V.
enum KvMode { kF32 = 0, kBF16 = 1, kI8K = 2 };

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

// MFMA operands are rounded with the hardware converter (v_cvt_pk_bf16_f32,
// round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)f[j];
  return r;
}

// ------------------------------------------------- asynchronous LDS staging
// A buffer resource over `bytes` bytes at base; reads past the end return
// zeros.  Copies into LDS use the MUBUF LDS-DMA form (buffer_load_dwordx4 ...
// lds), whose completion the compiler tracks on vmcnt alone: with the FLAT
// form (global_load_lds) it must assume the copy may also count on lgkmcnt,
// and while one is in flight every wait for an LDS read becomes a wait for
// all of them.
constexpr int kBufferConfig = 0x00020000;  // gfx9 dword 3: 32-bit data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferConfig);
}

// One wave instruction: lane l copies the 16 bytes at byte offset voffset
// (its own) of the resource to LDS address lds + 16 l (lds wave-uniform).
// 16-byte load marked non-temporal: data that is read once per call (the
// decode's streamed cache) need not displace reusable lines.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t rs, void* lds, int voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)lds, 16,
                                           voffset, 0, 0, 0);
}

// s_waitcnt vmcnt(0) through the builtin (not inline asm), so the compiler's
// own wait tracking sees it.  gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }
// s_waitcnt lgkmcnt(0): vmcnt 63, expcnt 7, lgkmcnt 0.
__device__ __forceinline__ void wait_lgkm() { __builtin_amdgcn_s_waitcnt(0xC07F); }
// s_waitcnt vmcnt(N) for a compile-time N < 64 (vmcnt bits [3:0] and [15:14]).
template <int N>
__device__ __forceinline__ void wait_vmem_le() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
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

// Bitwise OR across the 64 lanes of a wavefront (every lane ends with it).
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) x |= (uint32_t)__shfl_xor((int)x, m, kWave);
  return x;
}

// ------------------------------------------------- non-finite cache values
// bf16 (low 16 bits of h) and f32 bit patterns whose exponent is all ones:
// NaN or an infinity.
__device__ __forceinline__ bool bf16_nonfinite(uint32_t h) { return (h & 0x7f80u) == 0x7f80u; }
__device__ __forceinline__ bool f32_nonfinite(uint32_t u) {
  return (u & 0x7f800000u) == 0x7f800000u;
}

// The V cache's value at position p, dim d of one (session, KV head) slab, as
// f32 (plain loads: for the rare paths that add non-finite values back).
template <bool BF16>
__device__ __forceinline__ float v_at(const void* slab, int p, int d, int D) {
  if constexpr (BF16) {
    const uint16_t* s = reinterpret_cast<const uint16_t*>(slab);
    return __uint_as_float((uint32_t)s[((size_t)vbf16_group(p) * D + d) * 8 + vbf16_slot(p)] << 16);
  } else {
    const float* s = reinterpret_cast<const float*>(slab);
    return s[vf32_vec_index(p, d, D) * 4 + (p & 3)];
  }
}

// Class codes of a non-finite cache value: 1 +inf, 2 -inf, 3 NaN.  Terms
// w * v of such values summed into one accumulator combine by OR (+inf and
// -inf give NaN, as does NaN with anything).  A class table of a tile holds
// 2 bits per (position, dim): word p * D / 16 + d / 16, bits 2 (d % 16).
__device__ __forceinline__ uint32_t class_bf16(uint32_t h) {
  return (h & 0x7fu) != 0 ? 3u : ((h & 0x8000u) ? 2u : 1u);
}
__device__ __forceinline__ uint32_t class_f32(uint32_t u) {
  return (u & 0x7fffffu) != 0 ? 3u : ((u & 0x80000000u) ? 2u : 1u);
}
// Widens a byte of four class codes to NaN (3) where a code is set: a zero
// weight times an infinity is NaN.
__device__ __forceinline__ uint32_t all_nan(uint32_t byte) {
  return ((byte | (byte >> 1)) & 0x55u) * 3u;
}

// Adds the classes cls (2 bits per value of v: value i at bits 2 i) to the
// accumulator values: + inf, - inf or NaN.
template <int N, typename V>
__device__ __forceinline__ void apply_classes(uint32_t cls, V& v, int i0) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t c = (cls >> (2 * i)) & 3u;
    const float add = c == 1u ? INFINITY : (c == 2u ? -INFINITY : __builtin_nanf(""));
    v[i0 + i] = c != 0u ? v[i0 + i] + add : v[i0 + i];
  }
}

// ------------------------------------------------------- int8 K rows
// Symmetric int8 quantisation of one row (Karume v0.8.0 release notes,
// "Fixes": the activation-quantisation scale is amax times the f32 value of
// 1/127, in f32): s = amax * f32(1/127); code = round-half-even(x / s) (IEEE
// division), limited to +-127.  A row with a NaN gets s = NaN, an infinite
// one s = inf; rows whose s is 0 or not finite get codes 0 (their scores are
// then 0 * s).
constexpr float kInv127 = 1.0f / 127.0f;

// max |x| of the values seen so far, NaN once any of them was NaN
struct AbsMax {
  float m = 0.f;
  bool nan = false;
  __device__ __forceinline__ void add(float x) {
    nan = nan || (x != x);
    m = fmaxf(m, fabsf(x));
  }
  __device__ __forceinline__ float scale() const { return nan ? __builtin_nanf("") : m * kInv127; }
};

// A row's quantiser: its scale s and, when s and 1 / s are normal numbers,
// the correctly rounded reciprocal r = 1 / s (one division per row).  fast
// says whether quant_code_fast applies: for those scales, and for scales that
// are 0, NaN or infinite, whose codes are all 0 (r = 0 gives 0 for every
// finite value; a NaN or infinite value clears ok).  Only finite nonzero
// scales outside [2^-125, 2^125] need the division throughout.
struct RowQuant {
  float s, r;
  bool fast;
  __device__ __forceinline__ explicit RowQuant(float s_) : s(s_) {
    const bool normal = s_ >= 0x1p-125f && s_ <= 0x1p125f;
    fast = normal || !(s_ > 0.f) || !(s_ <= 3.402823466e38f);
    r = normal ? __fdiv_rn(1.f, s_) : 0.f;
  }
};

// rint of the IEEE f32 quotient x / s, limited to +-127.
__device__ __forceinline__ int quant_code(float x, const RowQuant& q) {
  if (!(q.s > 0.f) || !(q.s <= 3.402823466e38f)) return 0;  // 0, NaN or inf
  const float c = rintf(__fdiv_rn(x, q.s));
  return (int)fminf(fmaxf(c, -127.f), 127.f);
}

// Four codes (one little-endian word) without the division, valid while ok
// stays true.  The quotient's rounding can only change rint near a
// half-integer, so the product t = x * r (relative error below 2^-23: r's
// rounding and the product's) decides wherever it lies farther than
// |t| 2^-20 + 2^-22 from every half-integer h: then x / s, its f32 rounding
// and t all lie on t's side of h and round to the same integer (the absolute
// 2^-22 covers the rounding of fract(t) - 1/2).  About one value in 10^4
// clears ok; callers then redo the codes with pack_codes4 for the whole wave
// (one uniform branch), so the result is the division's bit for bit.  ok must
// start as q.fast (false for finite nonzero scales outside [2^-125, 2^125]).
__device__ __forceinline__ uint32_t pack_codes4_fast(float a, float b, float c, float d,
                                                     const RowQuant& q, bool& ok) {
  const float x[4] = {a, b, c, d};
  int k[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float t = x[i] * q.r;
    const float f = __builtin_amdgcn_fractf(t) - 0.5f;
    ok = ok && fabsf(f) > fmaf(fabsf(t), 0x1p-20f, 0x1p-22f);
    k[i] = (int)__builtin_amdgcn_fmed3f(rintf(t), -127.f, 127.f);
  }
  // low bytes of k0, k1 and of k2, k3, then the two halves
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)k[1], (uint32_t)k[0], 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)k[3], (uint32_t)k[2], 0x0c0c0400u);
  return lo | (hi << 16);
}

// Four codes packed little-endian into one 32-bit word.
__device__ __forceinline__ uint32_t pack_codes4(float a, float b, float c, float d,
                                                const RowQuant& q) {
  return (uint32_t)(quant_code(a, q) & 0xff) | ((uint32_t)(quant_code(b, q) & 0xff) << 8) |
         ((uint32_t)(quant_code(c, q) & 0xff) << 16) | ((uint32_t)(quant_code(d, q) & 0xff) << 24);
}

}  // namespace ka
