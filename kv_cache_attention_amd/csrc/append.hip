// KV append: new f32 rows [B][R][Hkv][D] -> cache positions start..start+R-1.
//
// One thread produces one 16-byte cache vector, so every store is a full
// 16-byte store except where a V vector (which spans 4 or 8 positions) is
// only partly covered by the appended range; there the covered elements are
// stored one by one and the rest of the vector is left untouched.
#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

template <bool BF16>
__global__ __launch_bounds__(256) void append_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache,
    const float* __restrict__ k_new, const float* __restrict__ v_new,
    int Hkv, int D, int C, int start, int R,
    long long n_k_vecs, long long n_v_vecs, int v_groups_per_slab, int v_group0) {
  constexpr int E = Elem<BF16>::E;
  const int cpr = D / E;  // K vectors per row
  long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  for (long long i = tid; i < n_k_vecs + n_v_vecs; i += stride) {
    if (i < n_k_vecs) {
      // K vector: (b, g, row, c) with c innermost
      const int c = (int)(i % cpr);
      long long t = i / cpr;
      const int g = (int)(t % Hkv);
      t /= Hkv;
      const int row = (int)(t % R);
      const int b = (int)(t / R);
      const int j = start + row;
      const float* src = k_new + (((size_t)b * R + row) * Hkv + g) * D + c * E;
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;  // elements
      const size_t vi = k_vec_index(j, c, D, E);
      if constexpr (BF16) {
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 bq = *reinterpret_cast<const float4*>(src + 4);
        uint4 o;
        o.x = pack_bf16x2(a.x, a.y);
        o.y = pack_bf16x2(a.z, a.w);
        o.z = pack_bf16x2(bq.x, bq.y);
        o.w = pack_bf16x2(bq.z, bq.w);
        reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_cache) + slab)[vi] = o;
      } else {
        const float4 a = *reinterpret_cast<const float4*>(src);
        reinterpret_cast<float4*>(reinterpret_cast<float*>(k_cache) + slab)[vi] = a;
      }
    } else {
      // V vector: (b, g, group, d) with d innermost; a group spans E positions
      const long long iv = i - n_k_vecs;
      const int d = (int)(iv % D);
      long long t = iv / D;
      const int gi = (int)(t % v_groups_per_slab) + v_group0;
      t /= v_groups_per_slab;
      const int g = (int)(t % Hkv);
      const int b = (int)(t / Hkv);
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;
      float vals[E];
      bool have[E];
      bool all = true;
#pragma unroll
      for (int s = 0; s < E; ++s) {
        int j;
        if constexpr (BF16) j = vbf16_pos(gi >> 2, gi & 3, s);
        else j = gi * 4 + s;
        const int row = j - start;
        have[s] = row >= 0 && row < R;
        all = all && have[s];
        vals[s] = have[s] ? v_new[(((size_t)b * R + row) * Hkv + g) * D + d] : 0.f;
      }
      const size_t vi = (size_t)gi * D + d;
      if constexpr (BF16) {
        uint16_t* base = reinterpret_cast<uint16_t*>(v_cache) + slab;
        if (all) {
          uint4 o;
          o.x = pack_bf16x2(vals[0], vals[1]);
          o.y = pack_bf16x2(vals[2], vals[3]);
          o.z = pack_bf16x2(vals[4], vals[5]);
          o.w = pack_bf16x2(vals[6], vals[7]);
          reinterpret_cast<uint4*>(base)[vi] = o;
        } else {
#pragma unroll
          for (int s = 0; s < E; ++s)
            if (have[s]) base[vi * 8 + s] = (uint16_t)f32_to_bf16_bits(vals[s]);
        }
      } else {
        float* base = reinterpret_cast<float*>(v_cache) + slab;
        if (all) {
          reinterpret_cast<float4*>(base)[vi] = make_float4(vals[0], vals[1], vals[2], vals[3]);
        } else {
#pragma unroll
          for (int s = 0; s < E; ++s)
            if (have[s]) base[vi * 4 + s] = vals[s];
        }
      }
    }
  }
}

hipError_t launch_append(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                         const float* v_new, int start, int R, hipStream_t stream) {
  const bool bf16 = s.kv_dtype == 1;
  const int E = bf16 ? 8 : 4;
  const long long n_k = (long long)s.batch * R * s.num_kv_heads * (s.head_dim / E);
  // V groups (of E positions) overlapping [start, start + R)
  int g0, g1;
  if (bf16) {
    // groups are not contiguous in position within a 32-block: cover whole blocks
    g0 = (start >> 5) * 4;
    g1 = ((start + R - 1) >> 5) * 4 + 4;
  } else {
    g0 = start >> 2;
    g1 = ((start + R - 1) >> 2) + 1;
  }
  const int ng = g1 - g0;
  const long long n_v = (long long)s.batch * s.num_kv_heads * ng * s.head_dim;
  const long long total = n_k + n_v;
  const int threads = 256;
  long long blocks = (total + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  if (bf16)
    hipLaunchKernelGGL(append_kernel<true>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       k_cache, v_cache, k_new, v_new, s.num_kv_heads, s.head_dim, s.capacity,
                       start, R, n_k, n_v, ng, g0);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3((unsigned)blocks), dim3(threads), 0, stream,
                       k_cache, v_cache, k_new, v_new, s.num_kv_heads, s.head_dim, s.capacity,
                       start, R, n_k, n_v, ng, g0);
  return hipGetLastError();
}

// One new row per session at its own position (the decode step's append):
// k_new / v_new [B][Hkv][D] f32 -> cache position pos[b].  Thread i writes
// one K vector or one V element (a V vector spans E positions, so only the
// row's own element of it is stored).
template <bool BF16>
__global__ __launch_bounds__(256) void append_row_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache, const float* __restrict__ k_new,
    const float* __restrict__ v_new, const CtxArg pos, int b0, int nb, int Hkv, int D, int C) {
  constexpr int E = Elem<BF16>::E;
  const int cpr = D / E;
  const long long nk = (long long)nb * Hkv * cpr, nv = (long long)nb * Hkv * D;
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < nk + nv;
       i += (long long)gridDim.x * blockDim.x) {
    if (i < nk) {
      const int c = (int)(i % cpr);
      const long long t = i / cpr;
      const int g = (int)(t % Hkv), bl = (int)(t / Hkv), b = b0 + bl;
      const int j = pos.ctx[bl];
      const float* src = k_new + ((size_t)b * Hkv + g) * D + c * E;
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;
      const size_t vi = k_vec_index(j, c, D, E);
      if constexpr (BF16) {
        const float4 a = *reinterpret_cast<const float4*>(src);
        const float4 bq = *reinterpret_cast<const float4*>(src + 4);
        uint4 o;
        o.x = pack_bf16x2(a.x, a.y);
        o.y = pack_bf16x2(a.z, a.w);
        o.z = pack_bf16x2(bq.x, bq.y);
        o.w = pack_bf16x2(bq.z, bq.w);
        reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_cache) + slab)[vi] = o;
      } else {
        reinterpret_cast<float4*>(reinterpret_cast<float*>(k_cache) + slab)[vi] =
            *reinterpret_cast<const float4*>(src);
      }
    } else {
      const long long iv = i - nk;
      const int d = (int)(iv % D);
      const long long t = iv / D;
      const int g = (int)(t % Hkv), bl = (int)(t / Hkv), b = b0 + bl;
      const int j = pos.ctx[bl];
      const float x = v_new[((size_t)b * Hkv + g) * D + d];
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;
      if constexpr (BF16) {
        uint16_t* base = reinterpret_cast<uint16_t*>(v_cache) + slab;
        base[((size_t)vbf16_group(j) * D + d) * 8 + vbf16_slot(j)] = (uint16_t)f32_to_bf16_bits(x);
      } else {
        float* base = reinterpret_cast<float*>(v_cache) + slab;
        base[vf32_vec_index(j, d, D) * 4 + (j & 3)] = x;
      }
    }
  }
}

hipError_t launch_append_rows(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                              const float* v_new, const CtxArg& pos, int b0, int nb,
                              hipStream_t stream) {
  const int E = s.kv_dtype == 1 ? 8 : 4;
  const long long total = (long long)nb * s.num_kv_heads * (s.head_dim / E + s.head_dim);
  long long blocks = (total + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (s.kv_dtype == 1)
    hipLaunchKernelGGL(append_row_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       k_cache, v_cache, k_new, v_new, pos, b0, nb, s.num_kv_heads, s.head_dim,
                       s.capacity);
  else
    hipLaunchKernelGGL(append_row_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, stream,
                       k_cache, v_cache, k_new, v_new, pos, b0, nb, s.num_kv_heads, s.head_dim,
                       s.capacity);
  return hipGetLastError();
}

}  // namespace ka
