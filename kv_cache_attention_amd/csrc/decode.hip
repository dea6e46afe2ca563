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
#include <type_traits>

#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

namespace {

constexpr int kUnit = 16;      // positions per wave work unit
constexpr int kWaves = 4;      // waves per workgroup
constexpr int kTargetWgs = 512;
constexpr int kMaxSplits = 1024;
constexpr int kSplitWavesPerEu = 2;  // register budget: 168 VGPRs, 12 waves per CU

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Position of lane-slot kk of unit u: units are 16 consecutive positions.
// With bf16 storage unit u is half s = u % 2 of 32-block u / 2, i.e. V groups
// 2 s and 2 s + 1 of that block.
__device__ __forceinline__ int unit_pos(int u, int kk) { return u * kUnit + kk; }
__device__ __forceinline__ int unit_last_pos(int u) { return u * kUnit + kUnit - 1; }
__host__ __device__ __forceinline__ int units_for(int ctx) { return (ctx + kUnit - 1) / kUnit; }

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

// K / V registers of one unit for one lane
template <int D, bool BF16>
struct UnitRegs {
  static constexpr int E = Elem<BF16>::E;
  static constexpr int NCH = D / (4 * E);   // K vectors: a quarter of D of one position
  static constexpr int ND = D / 64;         // value-stage dims per lane
  static constexpr int NG = kUnit / E;      // V vectors per dim per unit
  uint4 k[NCH];
  uint4 v[NG][ND];
};

template <int D, bool BF16>
__device__ __forceinline__ void load_unit_k(UnitRegs<D, BF16>& r, int u, int lane,
                                            const typename Elem<BF16>::T* __restrict__ kc) {
  using R = UnitRegs<D, BF16>;
  constexpr int E = R::E;
  const int kk = lane & 15, qd = lane >> 4;
  const int pos = unit_pos(u, kk);
#pragma unroll
  for (int i = 0; i < R::NCH; ++i)
    r.k[i] = *reinterpret_cast<const uint4*>(kc + k_vec_index(pos, qd * R::NCH + i, D, E) * E);
}

template <int D, bool BF16>
__device__ __forceinline__ void load_unit_v(UnitRegs<D, BF16>& r, int u, int lane,
                                            const typename Elem<BF16>::T* __restrict__ vc) {
  using R = UnitRegs<D, BF16>;
  constexpr int E = R::E;
#pragma unroll
  for (int gi = 0; gi < R::NG; ++gi) {
    int grp;
    if constexpr (BF16) grp = ((u >> 1) << 2) + ((u & 1) << 1) + gi;
    else grp = u * R::NG + gi;
#pragma unroll
    for (int t = 0; t < R::ND; ++t)
      r.v[gi][t] = *reinterpret_cast<const uint4*>(vc + ((size_t)grp * D + lane + 64 * t) * E);
  }
}

// Scores, online softmax and value accumulation of one unit.
template <int D, int HPW, bool BF16>
__device__ __forceinline__ void process_unit(UnitRegs<D, BF16>& r, int u, int lane, int ctx,
                                             float sl2e, const typename Elem<BF16>::T* q_lds,
                                             typename Elem<BF16>::T* p_lds, float (&m_run)[HPW],
                                             float (&l_run)[HPW],
                                             float (&acc)[HPW][UnitRegs<D, BF16>::ND]) {
  using R = UnitRegs<D, BF16>;
  constexpr int NCH = R::NCH, ND = R::ND, NG = R::NG;
  const int kk = lane & 15, qd = lane >> 4;
  const int pos = unit_pos(u, kk);
  // ---- scores: partial dot over this lane's quarter of D, then 2 xor steps.
  // q is read from LDS per 16-byte chunk; the fence after each chunk keeps the
  // compiler from hoisting every chunk's q into registers at once.
  using QV = typename std::conditional<BF16, uint4, float4>::type;
  const QV* qb = reinterpret_cast<const QV*>(q_lds + qd * (D / 4));
  constexpr int QH = D / (sizeof(QV) / sizeof(typename Elem<BF16>::T));  // QV per head
  float s[HPW];
#pragma unroll
  for (int h = 0; h < HPW; ++h) s[h] = 0.f;
#pragma unroll
  for (int i = 0; i < NCH; ++i) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      const QV qc = qb[h * QH + i];
      float a = s[h];
      if constexpr (BF16) {
        a = dot2_bf16(r.k[i].x, qc.x, a);
        a = dot2_bf16(r.k[i].y, qc.y, a);
        a = dot2_bf16(r.k[i].z, qc.z, a);
        a = dot2_bf16(r.k[i].w, qc.w, a);
      } else {
        a = fmaf(__uint_as_float(r.k[i].x), qc.x, a);
        a = fmaf(__uint_as_float(r.k[i].y), qc.y, a);
        a = fmaf(__uint_as_float(r.k[i].z), qc.z, a);
        a = fmaf(__uint_as_float(r.k[i].w), qc.w, a);
      }
      s[h] = a;
    }
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    float a = s[h];
    a += xor_shfl(a, 16);
    a += xor_shfl(a, 32);
    s[h] = pos < ctx ? a * sl2e : -INFINITY;
  }
  // ---- online softmax over the unit (16-lane butterfly max)
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
    if constexpr (BF16) slot = ((kk >> 2) & 1) * 8 + (kk & 3) + 4 * ((kk >> 3) & 1);
    else slot = kk;
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      if constexpr (BF16) p_lds[h * kUnit + slot] = (uint16_t)f32_to_bf16_bits(p[h]);
      else p_lds[h * kUnit + slot] = p[h];
    }
  }
  wave_lds_sync();
  // ---- positions at or beyond ctx may hold anything: zero their values
  if (unit_last_pos(u) >= ctx) {
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
        r.v[gi][t].x &= keep[0];
        r.v[gi][t].y &= keep[1];
        r.v[gi][t].z &= keep[2];
        r.v[gi][t].w &= keep[3];
      }
    }
  }
  // ---- values: acc[h][t] += sum over the unit's positions of p * v
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int h = 0; h < HPW; ++h) {
      if constexpr (BF16) {
        const uint4 pp = *reinterpret_cast<const uint4*>(p_lds + h * kUnit + gi * 8);
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          float a = acc[h][t];
          a = dot2_bf16(r.v[gi][t].x, pp.x, a);
          a = dot2_bf16(r.v[gi][t].y, pp.y, a);
          a = dot2_bf16(r.v[gi][t].z, pp.z, a);
          a = dot2_bf16(r.v[gi][t].w, pp.w, a);
          acc[h][t] = a;
        }
      } else {
        const float4 pp = *reinterpret_cast<const float4*>(p_lds + h * kUnit + gi * 4);
#pragma unroll
        for (int t = 0; t < ND; ++t) {
          float a = acc[h][t];
          a = fmaf(pp.x, __uint_as_float(r.v[gi][t].x), a);
          a = fmaf(pp.y, __uint_as_float(r.v[gi][t].y), a);
          a = fmaf(pp.z, __uint_as_float(r.v[gi][t].z), a);
          a = fmaf(pp.w, __uint_as_float(r.v[gi][t].w), a);
          acc[h][t] = a;
        }
      }
    }
  }
  wave_lds_sync();
}

template <int D, int HPW, bool BF16>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kSplitWavesPerEu)))
void decode_split_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    float* __restrict__ part_ml, const CtxArg ctxa, int b0, int Hq, int Hkv, int HG, int C,
    int S, float sl2e) {
  using R = UnitRegs<D, BF16>;
  constexpr int ND = R::ND;
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

  const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;
  const T* kc = reinterpret_cast<const T*>(k_cache) + slab;
  const T* vc = reinterpret_cast<const T*>(v_cache) + slab;
  const int n_units = units_for(ctx);
  const int u0 = (int)((long long)split * n_units / S);
  const int u1 = (int)((long long)(split + 1) * n_units / S);

  // first unit's loads go out before q, so the two latencies overlap
  R ra;
  int u = u0 + w;
  if (u < u1) {
    load_unit_k<D, BF16>(ra, u, lane, kc);
    load_unit_v<D, BF16>(ra, u, lane, vc);
  }

  // ---- q -> LDS (bf16 with RNE, or f32 copy); all loads issued first
  constexpr int QV = HPW * D / 2 / 256 > 0 ? HPW * D / 2 / 256 : 1;
  float2 qv[QV];
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const int i = tid + 256 * j;
    if (i < HPW * D / 2) {
      const int h = (2 * i) / D, d = (2 * i) % D;
      qv[j] = *reinterpret_cast<const float2*>(q + ((size_t)b * Hq + h0 + h) * D + d);
    }
  }
#pragma unroll
  for (int j = 0; j < QV; ++j) {
    const int i = tid + 256 * j;
    if (i < HPW * D / 2) {
      if constexpr (BF16) {
        reinterpret_cast<uint32_t*>(sm.q)[i] = pack_bf16x2(qv[j].x, qv[j].y);
      } else {
        sm.q[2 * i] = qv[j].x;
        sm.q[2 * i + 1] = qv[j].y;
      }
    }
  }
  __syncthreads();

  float m_run[HPW], l_run[HPW], acc[HPW][ND];
#pragma unroll
  for (int h = 0; h < HPW; ++h) {
    m_run[h] = -INFINITY;
    l_run[h] = 0.f;
#pragma unroll
    for (int t = 0; t < ND; ++t) acc[h][t] = 0.f;
  }

  // Latency is hidden by occupancy (several waves per SIMD, each with one
  // unit's loads in flight) rather than by a second register set per wave.
  bool first = true;
  for (; u < u1; u += kWaves) {
    if (!first) {
      load_unit_k<D, BF16>(ra, u, lane, kc);
      load_unit_v<D, BF16>(ra, u, lane, vc);
    }
    first = false;
    process_unit<D, HPW, BF16>(ra, u, lane, ctx, sl2e, sm.q, sm.p[w], m_run, l_run, acc);
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
      part[(((size_t)gq * S + split) * HPW + h) * D + d] = a;
      if (d == 0) {
        part_ml[(((size_t)gq * HPW + h) * S + split) * 2] = M;
        part_ml[(((size_t)gq * HPW + h) * S + split) * 2 + 1] = l;
      }
    }
  }
}

// Combines the S split partials of one (session, KV head, head group) for
// one head and 32 dims.  Thread (d, r) sums splits r, r + 8, ... with all its
// loads in flight; the eight partial sums are then added in a fixed order, so
// the result does not depend on timing.
template <int D, int HPW>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ part, const float* __restrict__ part_ml, float* __restrict__ out,
    int b0, int Hq, int Hkv, int HG, int S) {
  __shared__ float wgt[kMaxSplits];
  __shared__ float red[8][32];
  __shared__ float wmax[4], wsum[4];
  constexpr int NS = D / 32;
  const int h = blockIdx.x / NS, ds = blockIdx.x % NS;
  const int gh = blockIdx.y, bl = blockIdx.z, b = b0 + bl;
  const int g = gh / HG, hg = gh % HG;
  const int G = Hq / Hkv;
  const int gq = b * (Hkv * HG) + gh;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const float* ml = part_ml + ((size_t)gq * HPW + h) * S * 2;
  // M = max_s m_s over the block, then w_s = 2^(m_s - M), L = sum_s w_s l_s
  float M = -INFINITY;
  for (int s = tid; s < S; s += 256) M = fmaxf(M, ml[2 * s]);
  M = group_max<64>(M);
  if (lane == 0) wmax[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(wmax[0], wmax[1]), fmaxf(wmax[2], wmax[3]));
  float L = 0.f;
  for (int s = tid; s < S; s += 256) {
    const float ms = ml[2 * s];
    const float f = ms == -INFINITY ? 0.f : fast_exp2(ms - M);
    wgt[s] = f;
    L += f * ml[2 * s + 1];
  }
  L = group_sum<64>(L);
  if (lane == 0) wsum[w] = L;
  __syncthreads();
  L = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
  // weighted sum of the accumulators
  const int dl = tid & 31, r = tid >> 5;
  const int d = ds * 32 + dl;
  const float* pa = part + ((size_t)gq * S * HPW + h) * D + d;
  constexpr size_t PS = (size_t)HPW * D;
  float a = 0.f;
  int s = r;
  for (; s + 56 < S; s += 64) {
    float v[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = pa[(size_t)(s + 8 * j) * PS];
#pragma unroll
    for (int j = 0; j < 8; ++j) a += wgt[s + 8 * j] * v[j];
  }
  for (; s < S; s += 8) a += wgt[s] * pa[(size_t)s * PS];
  red[r][dl] = a;
  __syncthreads();
  if (r == 0) {
    const float t = ((red[0][dl] + red[1][dl]) + (red[2][dl] + red[3][dl])) +
                    ((red[4][dl] + red[5][dl]) + (red[6][dl] + red[7][dl]));
    out[((size_t)b * Hq + g * G + hg * HPW + h) * D + d] = t / L;
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
  float* part_ml = part + (size_t)s.batch * s.num_kv_heads * HG * S * HPW * D;
  hipLaunchKernelGGL((decode_split_kernel<D, HPW, BF16>), grid, dim3(256), 0, st, q, kc, vc, out,
                     part, part_ml, ca, b0, s.num_q_heads, s.num_kv_heads, HG, s.capacity, S,
                     sl2e);
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
    hipLaunchKernelGGL((decode_merge_kernel<D, H>), grid, dim3(256), 0, st, part,             \
                       part + (size_t)s.batch * s.num_kv_heads * HG * S * H * D, out, b0,     \
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
  const int units = units_for(max_ctx);
  const long long slabs = (long long)s.batch * s.num_kv_heads * p.head_groups;
  long long S = (kTargetWgs + slabs - 1) / slabs;
  const long long by_units = units / kWaves;  // at least one unit per wave
  if (S > by_units) S = by_units;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  p.splits = (int)S;
  p.workspace_bytes = p.splits == 1 ? 0
      : (size_t)slabs * p.splits * p.heads_per_wg * (s.head_dim + 2) * sizeof(float);
  // layout: acc [slab][S][HPW][D], then (m, l) [slab][HPW][S][2]
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
    if (S > 1) dispatch_merge<DD>(p.heads_per_wg,                                             \
                                  dim3(p.heads_per_wg * (DD / 32), s.num_kv_heads * HG, nb),   \
                                  stream, part,                                                \
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
