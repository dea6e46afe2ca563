// Split-context decode: one query row per session attends to ctx cached rows.
//
// Work decomposition.  The context of one (session, KV head) is cut into
// 16-position units.  A workgroup of four waves owns a contiguous range of
// units (one context split) and its waves take units round-robin, each wave
// keeping its own running max, sum and value accumulator.  Within a unit:
//
//  * scores: lane l handles position kk = l % 16 of the unit and a quarter
//    (l / 16) of the head dimension; its 16-byte K vectors are E consecutive
//    dims of one position, and the 16 positions of a quarter are adjacent in
//    the K layout, so each wave load is four 256-byte runs.  The partial dots
//    of the four quarters are summed with two cross-lane xor steps.
//  * softmax: the unit max is a 16-lane butterfly; weights are exp2 of
//    log2-domain scores (scale * log2 e folded into one multiply).
//  * values: lane l owns dims l + 64 t; each 16-byte V vector holds that dim
//    for E positions, so one wave load is a contiguous 1 KiB.  With bf16
//    storage two adjacent positions form a bf16 pair and v_dot2_f32_bf16
//    multiplies them with the matching pair of weights (rounded to bf16) in
//    one instruction, accumulating in f32.  f32 storage uses f32 FMAs.
//
// The four waves merge through LDS; with several splits each workgroup
// writes an unnormalised partial (m, l, acc) and a second kernel combines the
// splits in a fixed order, so the result is bitwise reproducible.
#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

namespace {

constexpr int kUnit = 16;      // positions per wave work unit
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kTargetWgs = 512;

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// position of lane-slot kk of unit u
template <bool BF16>
__device__ __forceinline__ int unit_pos(int u, int kk) {
  if constexpr (BF16) return ((u >> 1) << 5) + ((u & 1) << 3) + (kk & 7) + ((kk >> 3) << 4);
  else return u * kUnit + kk;
}

// last position of unit u (bf16 units interleave within 32-position blocks)
template <bool BF16>
__device__ __forceinline__ int unit_last_pos(int u) {
  if constexpr (BF16) return ((u >> 1) << 5) + ((u & 1) << 3) + 23;
  else return u * kUnit + kUnit - 1;
}

// Units covering positions 0 .. ctx-1: bf16 units come in pairs per
// 32-position block.
__host__ __device__ __forceinline__ int units_for(int ctx, bool bf16) {
  return bf16 ? 2 * ((ctx + 31) / 32) : (ctx + kUnit - 1) / kUnit;
}

template <int D, int HPW, bool BF16>
struct alignas(16) DecodeSmem {
  static constexpr int E = Elem<BF16>::E;
  // q: bf16 pairs or f32, [HPW][D]
  typename Elem<BF16>::T q[HPW * D];
  // per-wave weights of the current unit: [HPW][16 slots], in V-vector slot order
  typename Elem<BF16>::T p[kWaves][HPW * kUnit];
  float m[kWaves][HPW];
  float l[kWaves][HPW];
  float acc[kWaves][HPW * D];
};

template <int D, int HPW, bool BF16>
__global__ __launch_bounds__(256) void decode_split_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    const CtxArg ctxa, int b0, int Hq, int Hkv, int HG, int C, int S, float sl2e) {
  constexpr int E = Elem<BF16>::E;
  constexpr int NCH = D / (4 * E);   // K vectors per lane per unit (a quarter of D)
  constexpr int ND = D / 64;         // dims per lane in the value stage
  constexpr int NG = kUnit / E;      // V vectors (groups) per unit per dim
  using T = typename Elem<BF16>::T;
  __shared__ DecodeSmem<D, HPW, BF16> sm;

  const int split = blockIdx.x;
  const int gh = blockIdx.y;               // g * HG + hg
  const int g = gh / HG, hg = gh % HG;
  const int bl = blockIdx.z;
  const int b = b0 + bl;
  const int G = Hq / Hkv;
  const int h0 = g * G + hg * HPW;          // first query head served
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ctx = ctxa.ctx[bl];

  // ---- q -> LDS (bf16 with RNE, or f32 copy)
  for (int i = tid; i < HPW * D / 2; i += 256) {
    const int h = (2 * i) / D, d = (2 * i) % D;
    const float2 v = *reinterpret_cast<const float2*>(q + ((size_t)b * Hq + h0 + h) * D + d);
    if constexpr (BF16) {
      reinterpret_cast<uint32_t*>(sm.q)[i] = pack_bf16x2(v.x, v.y);
    } else {
      sm.q[2 * i] = v.x;
      sm.q[2 * i + 1] = v.y;
    }
  }
  __syncthreads();

  const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;
  const T* kc = reinterpret_cast<const T*>(k_cache) + slab;
  const T* vc = reinterpret_cast<const T*>(v_cache) + slab;

  const int n_units = units_for(ctx, BF16);
  const int u0 = (int)((long long)split * n_units / S);
  const int u1 = (int)((long long)(split + 1) * n_units / S);

  const int kk = lane & 15, qd = lane >> 4;

  float m_run[HPW], l_run[HPW], acc[HPW][ND];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int t = 0; t < ND; ++t) acc[h][t] = 0.f;
  }

  for (int u = u0 + w; u < u1; u += kWaves) {
    const int pos = unit_pos<BF16>(u, kk);
    // ---- issue K and V loads of the unit
    uint4 kv[NCH];
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      const int c = qd * NCH + i;
      kv[i] = *reinterpret_cast<const uint4*>(kc + k_vec_index(pos, c, D, E) * E);
    }
    uint4 vv[NG][ND];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      int grp;
      if constexpr (BF16) grp = ((u >> 1) << 2) + ((u & 1) << 1) + gi;
      else grp = u * NG + gi;
#pragma unroll
      for (int t = 0; t < ND; ++t)
        vv[gi][t] = *reinterpret_cast<const uint4*>(vc + ((size_t)grp * D + lane + 64 * t) * E);
    }
    // ---- scores (partial over this lane's quarter of D)
    float s[HPW];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      float a = 0.f;
      if constexpr (BF16) {
        const uint4* qv = reinterpret_cast<const uint4*>(sm.q + h * D + qd * (D / 4));
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const uint4 qq = qv[i];
          a = dot2_bf16(kv[i].x, qq.x, a);
          a = dot2_bf16(kv[i].y, qq.y, a);
          a = dot2_bf16(kv[i].z, qq.z, a);
          a = dot2_bf16(kv[i].w, qq.w, a);
        }
      } else {
        const float4* qv = reinterpret_cast<const float4*>(sm.q + h * D + qd * (D / 4));
#pragma unroll
        for (int i = 0; i < NCH; ++i) {
          const float4 qq = qv[i];
          a = fmaf(__uint_as_float(kv[i].x), qq.x, a);
          a = fmaf(__uint_as_float(kv[i].y), qq.y, a);
          a = fmaf(__uint_as_float(kv[i].z), qq.z, a);
          a = fmaf(__uint_as_float(kv[i].w), qq.w, a);
        }
      }
      a += xor_shfl(a, 16);
      a += xor_shfl(a, 32);
      s[h] = pos < ctx ? a * sl2e : -INFINITY;
    }
    const bool tail = unit_last_pos<BF16>(u) >= ctx;
    // ---- online softmax over the unit
    float p[HPW];
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const float mu = group_max<16>(s[h]);
      const float m_new = fmaxf(m_run[h], mu);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[h] - m_use);
      p[h] = fast_exp2(s[h] - m_use);
      l_run[h] = l_run[h] * alpha + p[h];
      m_run[h] = m_new;
#pragma unroll
      for (int t = 0; t < ND; ++t) acc[h][t] *= alpha;
    }
    // ---- weights -> LDS in V slot order (lanes 0..15 hold one copy)
    if (qd == 0) {
      int slot;
      if constexpr (BF16) slot = ((kk & 7) >> 2) * 8 + (kk & 3) + 4 * (kk >> 3);
      else slot = kk;
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        if constexpr (BF16) sm.p[w][h * kUnit + slot] = (uint16_t)f32_to_bf16_bits(p[h]);
        else sm.p[w][h * kUnit + slot] = p[h];
      }
    }
    wave_lds_sync();
    // positions at or beyond ctx may hold anything: zero their values
    if (tail) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        uint32_t keep[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (BF16) {
            const int sg = ((u & 1) << 1) + gi;
            const int p0 = vbf16_pos(u >> 1, sg, 2 * e), p1 = vbf16_pos(u >> 1, sg, 2 * e + 1);
            keep[e] = (p0 < ctx ? 0x0000ffffu : 0u) | (p1 < ctx ? 0xffff0000u : 0u);
          } else {
            keep[e] = (u * kUnit + gi * 4 + e) < ctx ? 0xffffffffu : 0u;
          }
        }
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          vv[gi][t].x &= keep[0];
          vv[gi][t].y &= keep[1];
          vv[gi][t].z &= keep[2];
          vv[gi][t].w &= keep[3];
        }
      }
    }
    // ---- values
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
      for (int h = 0; h < HPW; ++h) {
        if constexpr (BF16) {
          const uint4 pp = *reinterpret_cast<const uint4*>(&sm.p[w][h * kUnit + gi * 8]);
#pragma unroll
          for (int t = 0; t < ND; ++t) {
            float a = acc[h][t];
            a = dot2_bf16(vv[gi][t].x, pp.x, a);
            a = dot2_bf16(vv[gi][t].y, pp.y, a);
            a = dot2_bf16(vv[gi][t].z, pp.z, a);
            a = dot2_bf16(vv[gi][t].w, pp.w, a);
            acc[h][t] = a;
          }
        } else {
          const float4 pp = *reinterpret_cast<const float4*>(&sm.p[w][h * kUnit + gi * 4]);
#pragma unroll
          for (int t = 0; t < ND; ++t) {
            float a = acc[h][t];
            a = fmaf(pp.x, __uint_as_float(vv[gi][t].x), a);
            a = fmaf(pp.y, __uint_as_float(vv[gi][t].y), a);
            a = fmaf(pp.z, __uint_as_float(vv[gi][t].z), a);
            a = fmaf(pp.w, __uint_as_float(vv[gi][t].w), a);
            acc[h][t] = a;
          }
        }
      }
    }
    wave_lds_sync();
  }

  // ---- merge the four waves
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    const float lt = group_sum<16>(l_run[h]);
    if (lane == 0) {
      sm.m[w][h] = m_run[h];
      sm.l[w][h] = lt;
    }
#pragma unroll
    for (int t = 0; t < ND; ++t) sm.acc[w][h * D + lane + 64 * t] = acc[h][t];
  }
  __syncthreads();
  const int gq = b * (Hkv * HG) + gh;  // partial slot of (b, g, hg)
  for (int i = tid; i < HPW * D; i += 256) {
    const int h = i / D, d = i % D;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][h]);
    float a = 0.f, l = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = sm.m[ww][h] == -INFINITY ? 0.f : fast_exp2(sm.m[ww][h] - M);
      a += f * sm.acc[ww][i];
      l += f * sm.l[ww][h];
    }
    if (S == 1) {
      out[((size_t)b * Hq + h0 + h) * D + d] = a / l;
    } else {
      float* pa = part + ((size_t)gq * S + split) * HPW * (D + 2);
      pa[h * (D + 2) + 2 + d] = a;
      if (d == 0) {
        pa[h * (D + 2)] = M;
        pa[h * (D + 2) + 1] = l;
      }
    }
  }
}

// Combines the S split partials of one (session, KV head, head group).
template <int D, int HPW>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ part, float* __restrict__ out, int b0, int Hq, int Hkv, int HG,
    int S) {
  __shared__ float wgt[HPW * 1024];
  __shared__ float Ms[HPW];
  const int gh = blockIdx.x, bl = blockIdx.y, b = b0 + bl;
  const int g = gh / HG, hg = gh % HG;
  const int G = Hq / Hkv;
  const int h0 = g * G + hg * HPW;
  const int gq = b * (Hkv * HG) + gh;
  const float* pb = part + (size_t)gq * S * HPW * (D + 2);
  const int tid = threadIdx.x;
  // per head: M = max_s m_s, then w_s = 2^(m_s - M) in a fixed order
  for (int h = tid >> 6; h < HPW; h += 4) {
    const int ln = tid & 63;
    float M = -INFINITY;
    for (int s = ln; s < S; s += 64) M = fmaxf(M, pb[((size_t)s * HPW + h) * (D + 2)]);
    M = group_max<64>(M);
    float L = 0.f;
    for (int s = ln; s < S; s += 64) {
      const float* e = pb + ((size_t)s * HPW + h) * (D + 2);
      const float f = e[0] == -INFINITY ? 0.f : fast_exp2(e[0] - M);
      wgt[h * 1024 + s] = f;
      L += f * e[1];
    }
    L = group_sum<64>(L);
    if (ln == 0) Ms[h] = L;
  }
  __syncthreads();
  for (int i = tid; i < HPW * D; i += 256) {
    const int h = i / D, d = i % D;
    float a = 0.f;
    for (int s = 0; s < S; ++s) a += wgt[h * 1024 + s] * pb[((size_t)s * HPW + h) * (D + 2) + 2 + d];
    out[((size_t)b * Hq + h0 + h) * D + d] = a / Ms[h];
  }
}

int heads_per_wg(int G) {
  if (G % 8 == 0) return 8;
  if (G % 4 == 0) return 4;
  if (G % 2 == 0) return 2;
  return 1;
}

template <int D, int HPW, bool BF16>
void launch_split(dim3 grid, hipStream_t st, const float* q, const void* kc, const void* vc,
                  float* out, float* part, const CtxArg& ca, int b0, const Shape& s, int HG,
                  int S, float sl2e) {
  hipLaunchKernelGGL((decode_split_kernel<D, HPW, BF16>), grid, dim3(256), 0, st, q, kc, vc, out,
                     part, ca, b0, s.num_q_heads, s.num_kv_heads, HG, s.capacity, S, sl2e);
}

template <int D, bool BF16>
void dispatch_hpw(int hpw, dim3 grid, hipStream_t st, const float* q, const void* kc,
                  const void* vc, float* out, float* part, const CtxArg& ca, int b0,
                  const Shape& s, int HG, int S, float sl2e) {
  switch (hpw) {
    case 8: launch_split<D, 8, BF16>(grid, st, q, kc, vc, out, part, ca, b0, s, HG, S, sl2e); break;
    case 4: launch_split<D, 4, BF16>(grid, st, q, kc, vc, out, part, ca, b0, s, HG, S, sl2e); break;
    case 2: launch_split<D, 2, BF16>(grid, st, q, kc, vc, out, part, ca, b0, s, HG, S, sl2e); break;
    default: launch_split<D, 1, BF16>(grid, st, q, kc, vc, out, part, ca, b0, s, HG, S, sl2e); break;
  }
}

template <int D>
void dispatch_merge(int hpw, dim3 grid, hipStream_t st, const float* part, float* out, int b0,
                    const Shape& s, int HG, int S) {
  switch (hpw) {
#define KA_MERGE(H)                                                                            \
  case H:                                                                                      \
    hipLaunchKernelGGL((decode_merge_kernel<D, H>), grid, dim3(256), 0, st, part, out, b0,    \
                       s.num_q_heads, s.num_kv_heads, HG, S);                                  \
    break;
    KA_MERGE(8) KA_MERGE(4) KA_MERGE(2) KA_MERGE(1)
#undef KA_MERGE
  }
}

}  // namespace

DecodePlan plan_decode(const Shape& s, int max_ctx) {
  DecodePlan p;
  const int G = s.num_q_heads / s.num_kv_heads;
  p.heads_per_wg = heads_per_wg(G);
  p.head_groups = G / p.heads_per_wg;
  const int units = units_for(max_ctx, s.kv_dtype == 1);
  const long long slabs = (long long)s.batch * s.num_kv_heads * p.head_groups;
  long long S = (kTargetWgs + slabs - 1) / slabs;
  const long long by_units = units / kWaves;  // at least one unit per wave
  if (S > by_units) S = by_units;
  if (S > 1024) S = 1024;
  if (S < 1) S = 1;
  p.splits = (int)S;
  p.workspace_bytes = p.splits == 1 ? 0
      : (size_t)slabs * p.splits * p.heads_per_wg * (s.head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_decode(const Shape& s, const DecodePlan& p, const float* q,
                         const void* k_cache, const void* v_cache, float* out,
                         const int32_t* ctx_host, float scale, void* workspace,
                         hipStream_t stream) {
  const bool bf16 = s.kv_dtype == 1;
  const float sl2e = scale * kLog2e;
  const int HG = p.head_groups, S = p.splits;
  float* part = reinterpret_cast<float*>(workspace);
  for (int b0 = 0; b0 < s.batch; b0 += kMaxDecodeBatchPerLaunch) {
    const int nb = s.batch - b0 < kMaxDecodeBatchPerLaunch ? s.batch - b0 : kMaxDecodeBatchPerLaunch;
    CtxArg ca;
    for (int i = 0; i < kMaxDecodeBatchPerLaunch; ++i) ca.ctx[i] = i < nb ? ctx_host[b0 + i] : 0;
    dim3 grid(S, s.num_kv_heads * HG, nb);
    switch (s.head_dim) {
#define KA_D(DD)                                                                               \
  case DD:                                                                                     \
    if (bf16) dispatch_hpw<DD, true>(p.heads_per_wg, grid, stream, q, k_cache, v_cache, out,  \
                                     part, ca, b0, s, HG, S, sl2e);                            \
    else dispatch_hpw<DD, false>(p.heads_per_wg, grid, stream, q, k_cache, v_cache, out, part, \
                                 ca, b0, s, HG, S, sl2e);                                      \
    if (S > 1) dispatch_merge<DD>(p.heads_per_wg, dim3(s.num_kv_heads * HG, nb), stream, part, \
                                  out, b0, s, HG, S);                                          \
    break;
      KA_D(64) KA_D(128) KA_D(256)
#undef KA_D
      default: return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace ka
