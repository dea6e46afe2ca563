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
constexpr float kRescaleSlack = 8.f;  // log2 units (MFMA path)

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
  // the decode step's new K and V rows (f32), for the wave that owns them
  float row[2][D];
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
    r.k[i] = load_stream16(kc + k_vec_index(pos, qd * R::NCH + i, D, E) * E);
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
      r.v[gi][t] = load_stream16(vc + ((size_t)grp * D + lane + 64 * t) * E);
  }
}

// Scores, online softmax and value accumulation of one unit.  Once the
// scores have used the K registers, the K of unit next_u (if >= 0) is loaded
// into them.
template <int D, int HPW, bool BF16>
__device__ __forceinline__ void process_unit(UnitRegs<D, BF16>& r, int u, int lane, int ctx,
                                             float sl2e, const typename Elem<BF16>::T* q_lds,
                                             typename Elem<BF16>::T* p_lds, float (&m_run)[HPW],
                                             float (&l_run)[HPW],
                                             float (&acc)[HPW][UnitRegs<D, BF16>::ND],
                                             int next_u,
                                             const typename Elem<BF16>::T* __restrict__ kc) {
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
  // the next loads may not move above the last use of the K registers
  __builtin_amdgcn_sched_barrier(0);
  if (next_u >= 0) load_unit_k<D, BF16>(r, next_u, lane, kc);
  __builtin_amdgcn_sched_barrier(0);
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
    float* __restrict__ part_ml, const float* __restrict__ k_new, const float* __restrict__ v_new,
    const CtxArg ctxa, int b0, int Hq, int Hkv, int HG, int C, int S, float sl2e) {
  static_assert(!BF16, "bf16 caches decode on the MFMA kernel");
  using R = UnitRegs<D, BF16>;
  constexpr int ND = R::ND, NCH = R::NCH;
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

  // The decode step's new row (k_new / v_new, position ctx - 1): the wave
  // whose unit holds it loads it before anything else (the caller's last
  // kernel wrote it, so it may be far from this CU, and its latency should
  // run alongside the first unit's and q's), keeps it in LDS, stores it as
  // the append kernel would (an f32 copy; head group 0 of the slab only),
  // and takes its values in place of what its loads of that unit bring in,
  // so no wave waits on the store and no other wave reads that position.
  const int p_new = ctx - 1, u_new = p_new / kUnit;
  const bool owns_new = k_new != nullptr && u_new >= u0 && u_new < u1 &&
                        (u_new - u0) % kWaves == w;
  float4 nk = make_float4(0.f, 0.f, 0.f, 0.f);  // K dims 4 lane .. 4 lane + 3 (lanes below D / 4)
  float nv[ND];                                  // V dims lane + 64 t
#pragma unroll
  for (int t = 0; t < ND; ++t) nv[t] = 0.f;
  if (owns_new) {
    const float* kn = k_new + ((size_t)b * Hkv + g) * D;
    const float* vn = v_new + ((size_t)b * Hkv + g) * D;
    if (4 * lane < D) nk = *reinterpret_cast<const float4*>(kn + 4 * lane);
#pragma unroll
    for (int t = 0; t < ND; ++t) nv[t] = vn[lane + 64 * t];
  }
  auto take_new_row = [&](R& r) {
    if ((lane & 15) == (p_new & 15)) {  // this lane's K slices are of the new position
      const int qd = lane >> 4;
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const float4 x = *reinterpret_cast<const float4*>(&sm.row[0][4 * (qd * NCH + i)]);
        r.k[i] = make_uint4(__float_as_uint(x.x), __float_as_uint(x.y), __float_as_uint(x.z),
                            __float_as_uint(x.w));
      }
    }
    const int gi = (p_new & 15) >> 2, e = p_new & 3;  // V: group gi of the unit, slot e
#pragma unroll
    for (int t = 0; t < ND; ++t) {
      const uint32_t x = __float_as_uint(sm.row[1][lane + 64 * t]);
#pragma unroll
      for (int g2 = 0; g2 < R::NG; ++g2) {
        // a select per element (a skipped iteration became a runtime index
        // into a stack copy of the registers at D = 64)
        const bool sg = g2 == gi;
        r.v[g2][t].x = sg && e == 0 ? x : r.v[g2][t].x;
        r.v[g2][t].y = sg && e == 1 ? x : r.v[g2][t].y;
        r.v[g2][t].z = sg && e == 2 ? x : r.v[g2][t].z;
        r.v[g2][t].w = sg && e == 3 ? x : r.v[g2][t].w;
      }
    }
  };

  // The first unit's K, then q, then that unit's V: loads return in issue
  // order, so q reaches LDS, and the first scores start, while V is still
  // arriving (with q after V, both waited for the whole unit)
  R ra;
  int u = u0 + w;
  if (u < u1) load_unit_k<D, BF16>(ra, u, lane, kc);
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
  if (u < u1) load_unit_v<D, BF16>(ra, u, lane, vc);
  if (owns_new) {
    if (4 * lane < D) *reinterpret_cast<float4*>(&sm.row[0][4 * lane]) = nk;
#pragma unroll
    for (int t = 0; t < ND; ++t) sm.row[1][lane + 64 * t] = nv[t];
    if (hg == 0) {
      float* kw = reinterpret_cast<float*>(const_cast<void*>(k_cache)) + slab;
      float* vw = reinterpret_cast<float*>(const_cast<void*>(v_cache)) + slab;
      if (4 * lane < D) *reinterpret_cast<float4*>(kw + k_vec_index(p_new, lane, D, 4) * 4) = nk;
#pragma unroll
      for (int t = 0; t < ND; ++t)
        vw[vf32_vec_index(p_new, lane + 64 * t, D) * 4 + (p_new & 3)] = nv[t];
    }
    wave_lds_sync();
  }

  // ---- q -> LDS (bf16 with RNE, or f32 copy)
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

  // One register set per wave (the operands of a unit fill most of it): the
  // next unit's K goes into the K registers as soon as the scores have used
  // them, so it arrives during this unit's softmax and value product, and a
  // unit's V is loaded ahead of its scores; the other waves of the SIMD
  // cover the rest of the latency.  (Loading the next V at the end of a unit
  // instead made the compiler keep far more registers live: 129 -> 255 at
  // D = 64, spills at D = 256.)
  for (; u < u1; u += kWaves) {
    const int nu = u + kWaves;
    if (u != u0 + w) load_unit_v<D, BF16>(ra, u, lane, vc);  // the first unit's went out early
    if (owns_new && u == u_new) take_new_row(ra);
    process_unit<D, HPW, BF16>(ra, u, lane, ctx, sl2e, sm.q, sm.p[w], m_run, l_run, acc,
                               nu < u1 ? nu : -1, kc);
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
// one head and 32 dims.  Thread (d, r) takes splits r, r + 8, r + 16, ...:
// it loads the accumulators and (m, l) records of its first kMergeEarly
// splits before using any (every MFMA plan fits, so the merge waits on
// memory about once; the f32 plans' longer split lists follow in batches of
// kMergeTail), and sums them in its own frame; the eight threads of a dim then combine their
// (m, l, acc) through LDS in the fixed order r = 0 .. 7 (one barrier), so the
// result does not depend on timing.  A split that saw no key (l = 0) adds
// nothing; one whose sum is NaN (NaN scores, even with m = -inf) makes the
// result NaN.
constexpr int kMergeEarly = 32;
constexpr int kMergeTail = 16;

// NB: batches of 8 splits that every thread loads at once (8 NB >= S up to
// kMergeEarly batches; the host picks it from S).
template <int D, int NB>
__global__ __launch_bounds__(256) void decode_merge_kernel(
    const float* __restrict__ part, const float* __restrict__ part_ml, float* __restrict__ out,
    int b0, int Hq, int Hkv, int HG, int hpw, int S, int R) {
  __shared__ float red_a[8][32];
  __shared__ float red_m[8], red_l[8];
  constexpr int NS = D / 32;
  const int h = blockIdx.x / NS, ds = blockIdx.x % NS;
  const int gh = blockIdx.y, bl = blockIdx.z, b = b0 + bl;
  const int g = HG == 1 ? gh : gh / HG, hg = HG == 1 ? 0 : gh % HG;  // no division for one group
  const int G = Hq / Hkv;
  const int gq = b * (Hkv * HG) + gh;
  const int ph = hg * hpw + h;  // (row, head) pair of the group: row ph / G, head ph % G
  if (ph >= R * G) return;      // block-uniform: before the barrier
  const int tid = threadIdx.x;
  const float2* ml = reinterpret_cast<const float2*>(part_ml + ((size_t)gq * hpw + h) * S * 2);
  const int dl = tid & 31, r = tid >> 5;
  const int d = ds * 32 + dl;
  // a base common to the block and 32-bit offsets (s PS + d < 2^31: at most
  // 1024 splits of 16 heads of 256 dims)
  const float* pa = part + ((size_t)gq * S * hpw + h) * D;
  const int PS = hpw * D;
  // The loads first, all of them in flight together and with no condition
  // around them: a thread whose split of a batch is past the end loads split
  // S - 1 and its value is replaced afterwards.  (A per-thread or per-batch
  // condition around the loads lets the compiler copy a loaded register at
  // the join, waiting for that load before it issues the rest: a second
  // memory round trip.)
  float av[NB];
  float2 mlv[NB];
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const int s = min(r + 8 * k, S - 1);
    av[k] = pa[s * PS + d];
    mlv[k] = ml[s];
  }
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    const bool in = r + 8 * k < S;
    av[k] = in ? av[k] : 0.f;
    mlv[k] = in ? mlv[k] : make_float2(-INFINITY, 0.f);
  }
  float m = -INFINITY;
#pragma unroll
  for (int k = 0; k < NB; ++k) m = fmaxf(m, mlv[k].x);
  float l = 0.f, a = 0.f;
#pragma unroll
  for (int k = 0; k < NB; ++k) {
    if (mlv[k].y == 0.f) continue;
    const float f = fast_exp2(mlv[k].x - m);
    l += f * mlv[k].y;
    a += f * av[k];
  }
  // more than 8 kMergeEarly splits (f32 plans): further batches of kMergeTail
  // splits per thread, each batch's loads issued together, in a running
  // frame that moves to the batch's largest m
  for (int sb = 8 * NB; sb < S; sb += 8 * kMergeTail) {  // the same batches for all threads
    float bv[kMergeTail];
    float2 bml[kMergeTail];
#pragma unroll
    for (int k = 0; k < kMergeTail; ++k) {
      const int s = min(sb + r + 8 * k, S - 1);
      bv[k] = pa[s * PS + d];
      bml[k] = ml[s];
    }
#pragma unroll
    for (int k = 0; k < kMergeTail; ++k) {
      const bool in = sb + r + 8 * k < S;
      bv[k] = in ? bv[k] : 0.f;
      bml[k] = in ? bml[k] : make_float2(-INFINITY, 0.f);
    }
    float mb = m;
#pragma unroll
    for (int k = 0; k < kMergeTail; ++k) mb = fmaxf(mb, bml[k].x);
    if (mb > m) {
      const float f = fast_exp2(m - mb);  // 0 while m is -inf
      l *= f;
      a *= f;
      m = mb;
    }
#pragma unroll
    for (int k = 0; k < kMergeTail; ++k) {
      if (bml[k].y == 0.f) continue;
      const float f = fast_exp2(bml[k].x - m);
      l += f * bml[k].y;
      a += f * bv[k];
    }
  }
  red_a[r][dl] = a;
  if (dl == 0) {
    red_m[r] = m;
    red_l[r] = l;
  }
  __syncthreads();
  if (r != 0) return;
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < 8; ++j) M = fmaxf(M, red_m[j]);
  float A = 0.f, L = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (red_l[j] == 0.f) continue;
    const float f = fast_exp2(red_m[j] - M);
    A += f * red_a[j][dl];
    L += f * red_l[j];
  }
  const int prow = R == 1 ? 0 : ph / G, phead = R == 1 ? ph : ph % G;
  out[(((size_t)b * R + prow) * Hq + g * G + phead) * D + d] = A / L;
}

// ============================================================================
// bf16 caches: the decode step on MFMA (v_mfma_f32_16x16x32_bf16).
//
// One query row with hpw <= 16 heads is a prefill of one row: the heads are
// the MFMA columns.  The context is cut into 32-position tiles (one bf16 V
// block); the S workgroups of a (session, KV head) and their four waves each
// take every (4 S)-th tile.  A wave loads its MFMA
// operands straight from the cache into registers -- every K / V element is
// used by exactly one wave, so there is nothing for LDS to share -- two tiles
// ahead (64 KiB in flight per wave for D = 256).  Per tile (lane l: column
// l % 16, row group r = l / 16):
//   S^T = K . Q^T per 16-position block kb and 32-dim step ks: A = K[32 t +
//     16 kb + l % 16][32 ks + 8 r .. + 7] (16 bytes of the K layout), B = Q^T
//     (stationary; scale * log2 e folded in, rounded once to bf16).  The lane
//     then holds positions 32 t + 16 kb + 4 r + 0..3 of its column.
//   O^T += V^T . P^T per 16-dim block db: A = V group r at dim 16 db + l % 16
//     (16 bytes: 8 positions), B = the weights of those 8 positions for the
//     lane's column.  Group r = 2 s + h holds positions {16 s + 4 h + 0..3,
//     16 s + 8 + 4 h + 0..3}: a lane in the lower half (r < 2) owns the first
//     four in its own block-0 scores and finds the other four in the lane 32
//     above; a lane in the upper half owns the last four (block 1) and finds
//     the first four 32 below -- one v_permlane32_swap per register pair.
// The four waves merge through LDS; a workgroup writes its split's partial
// (or, alone, the output); a second kernel combines the splits.
// ============================================================================
constexpr int kDecTile = 32;  // positions per wave tile
// Buffer-load cache policy of the streamed K / V operands: non-temporal (NT).
constexpr int kStreamAux = 2;
constexpr int kDecCols = 16;  // MFMA columns = most heads per workgroup

// I8: int8 K codes (16 per 16-byte vector, so a score step covers 64 dims)
// with one f32 scale per position, scores on v_mfma_i32_16x16x64_i8.
template <int D, bool I8>
struct DecTile {
  static constexpr int NKS = I8 ? D / 64 : D / 32;  // score k-steps
  uint4 k[2][NKS];     // [position block kb][dim step ks]
  uint4 v[D / 16];     // [dim block db]
  float4 sk[I8 ? 2 : 1];  // I8: scales of positions 16 kb + 4 r + 0..3
};

template <int D, bool I8, bool ROWS>
__global__ __launch_bounds__(256) void decode_mfma_kernel(
    const float* __restrict__ q, void* k_cache, void* v_cache, float* __restrict__ out,
    float* __restrict__ part, float* __restrict__ part_ml, const float* __restrict__ k_new,
    const float* __restrict__ v_new, float* __restrict__ k_scales, const CtxArg ctxa,
    int b0, int nb, int Hq, int Hkv, int HG, int hpw, int C, int S, float sl2e, int R) {
  typedef __attribute__((ext_vector_type(4))) float v4f;
  typedef __attribute__((ext_vector_type(4))) int i32x4;
  constexpr int NKS = DecTile<D, I8>::NKS;
  constexpr int KE = I8 ? 16 : 8;  // K elements per 16-byte vector
  __shared__ float sacc[kWaves][kDecCols * D];
  __shared__ float wm[kWaves][kDecCols], wl[kWaves][kDecCols];

  // Work item i = ((session bl, KV head g, split) , head group hg), hg fastest.
  // One head group: item i is workgroup i.  Several: workgroups go to the 8
  // XCDs in turn, so workgroup x takes item (x % 8) per + x / 8 and each XCD
  // holds a contiguous run of items -- the head groups of a split together,
  // reading the same K / V lines through one L2.  Items past the end exit.
  // One head group: the grid is (split, KV head, session), read straight
  // from the block index, so the context length's load needs no other
  // argument first.
  int hg = 0, split, g, bl;
  if (HG > 1) {
    const int per = (int)((gridDim.x + 7) / 8);
    const int item = (blockIdx.x & 7) * per + (blockIdx.x >> 3);
    if (item >= nb * Hkv * S * HG) return;
    hg = item % HG;
    split = (item / HG) % S;
    const int gb = item / (HG * S);
    g = gb % Hkv;
    bl = gb / Hkv;
  } else {
    split = blockIdx.x;
    g = blockIdx.y;
    bl = blockIdx.z;
  }
  const int b = b0 + bl;
  const int gh = g * HG + hg;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lc = lane & 15, r = lane >> 4;
  const int ctx = ctxa.ctx[bl];
  const int nt = (ctx + kDecTile - 1) / kDecTile;
  // The slab's S * 4 waves take its tiles in turn (wave j: tiles j, j + NW,
  // j + 2 NW, ...), so at any moment they read one contiguous stretch of the
  // cache; a wave's tiles need no order (the softmax is online).
  const int NW = S * kWaves, j0 = split * kWaves + w;
  // Local tile counts from one division of the workgroup: with nt - 1 =
  // qn NW + rn, a wave j0 <= rn has qn + 1 tiles, one above it qn, and the
  // last tile (that of the decode step's new row) is wave rn's.
  const int qn = (nt - 1) / NW, rn = nt - 1 - qn * NW;
  const int t0 = 0, t1 = qn + (j0 <= rn ? 1 : 0);
  // whether the wave has a first and a second tile, without waiting for t1
  const bool has0 = j0 < nt, has1 = j0 + NW < nt;

  const size_t slab_bytes = (size_t)C * D * 2;                 // V (and bf16 K)
  const size_t k_slab_bytes = (size_t)C * D * (I8 ? 1 : 2);
  const size_t slab_i = (size_t)b * Hkv + g;
  const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(
      reinterpret_cast<const unsigned char*>(k_cache) + slab_i * k_slab_bytes, k_slab_bytes);
  const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(
      reinterpret_cast<const unsigned char*>(v_cache) + slab_i * slab_bytes, slab_bytes);
  const float* __restrict__ sk_row = I8 ? k_scales + slab_i * C : nullptr;

  // operand loads of this wave's i-th tile, tile j0 + i NW (K layout
  // [C/64][D/KE][64][KE], V [C/32][4][D][8]); every cache byte is read once per
  // step, so the loads are marked non-temporal
  auto load_k = [&](DecTile<D, I8>& x, int i) {
    const int t = j0 + i * NW;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int pos = kDecTile * t + 16 * kb + lc;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks)
        x.k[kb][ks] = __builtin_bit_cast(
            uint4, __builtin_amdgcn_raw_buffer_load_b128(
                       krs, (((pos >> 6) * (D / KE) + 4 * ks + r) * 64 + (pos & 63)) * 16, 0, kStreamAux));
      if constexpr (I8)
        x.sk[kb] = *reinterpret_cast<const float4*>(sk_row + kDecTile * t + 16 * kb + 4 * r);
    }
  };
  auto load_v = [&](DecTile<D, I8>& x, int i) {
    const int t = j0 + i * NW;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      x.v[db] = __builtin_bit_cast(
          uint4, __builtin_amdgcn_raw_buffer_load_b128(
                     vrs, ((4 * t + r) * D + 16 * db + lc) * 16, 0, kStreamAux));
  };
  auto load = [&](DecTile<D, I8>& x, int i) {
    load_k(x, i);
    load_v(x, i);
  };

  // The decode step's new row (position ctx - 1, given by k_new / v_new; its
  // handling is described below).  The wave that owns it loads it before
  // anything else: k_new and v_new come from the caller's last kernel and may
  // be far from this CU, and their latency should run alongside the tiles'
  // and q's, not after them (one 16K step with inputs not in cache: 17.9 us
  // with these loads after q, as the other inputs' latency allows).
  const int p_new = ctx - 1, t_new = p_new / kDecTile;
  const bool owns_new = k_new != nullptr && j0 == rn;  // t_new = nt - 1
  // K: lane l holds dims 8 l .. 8 l + 7 (bf16, lanes below D / 8) or 4 l ..
  // 4 l + 3 (int8-K, lanes below D / 4); V: dims l + 64 i
  float4 nk0 = make_float4(0.f, 0.f, 0.f, 0.f), nk1 = nk0;
  float nv[D / 64];
#pragma unroll
  for (int i = 0; i < D / 64; ++i) nv[i] = 0.f;
  if (owns_new) {
    const float* kn = k_new + ((size_t)b * Hkv + g) * D;
    const float* vn = v_new + ((size_t)b * Hkv + g) * D;
    if constexpr (I8) {
      if (4 * lane < D) nk0 = *reinterpret_cast<const float4*>(kn + 4 * lane);
    } else if (lane < D / 8) {
      nk0 = *reinterpret_cast<const float4*>(kn + 8 * lane);
      nk1 = *reinterpret_cast<const float4*>(kn + 8 * lane + 4);
    }
#pragma unroll
    for (int i = 0; i < D / 64; ++i) nv[i] = vn[lane + 64 * i];
  }

  // stationary Q^T: column lc is (row, head) pair pc = hg hpw + lc of the KV
  // group -- query row pc / G of the session's R rows (the last of which sits
  // at position ctx - 1), head g G + pc % G -- and zero past the pairs.  Its
  // keys are 0 .. lim.
  bf16x8 qreg[I8 ? 1 : D / 32];
  i32x4 qcode[I8 ? D / 64 : 1];  // I8: the column's codes, dims 64 ks + 16 r .. + 15
  float sq = 0.f;                // I8: the column's scale times scale * log2 e
  const int pc = hg * hpw + lc;
  const bool hv = lc < hpw && pc < R * G;
  // the column's query row and head (one row without ROWS: row 0, head pc)
  const int prow = ROWS ? (hv ? pc / G : 0) : 0, phead = ROWS ? (hv ? pc % G : 0) : (hv ? pc : 0);
  const int lim = ctx - R + prow;

  // The first tile's K, then this column's q (f32; converted or quantised
  // below), then that tile's V and the second tile.  Loads return in issue
  // order, so the first tile's scores wait for its K and q only and run
  // while its V arrives (with q issued after both tiles, they waited for
  // all of them: a 16K step 13.8 -> 12.5 us).  Lane (lc, r) takes the dims
  // of its MFMA operand: float4 n holds dims 32 (n / 2) + 8 r + 4 (n % 2)
  // (bf16) or 64 (n / 4) + 16 r + 4 (n % 4) (int8 codes).
  DecTile<D, I8> ta_, tb_;
  float4 qraw[D / 16];
  if (has0) load_k(ta_, t0);
  {
    const float* qp = q + (((size_t)b * R + prow) * Hq + g * G + phead) * D + (I8 ? 16 : 8) * r;
#pragma unroll
    for (int n = 0; n < D / 16; ++n) {
      const int off = I8 ? 64 * (n >> 2) + 4 * (n & 3) : 32 * (n >> 1) + 4 * (n & 1);
      qraw[n] = hv ? *reinterpret_cast<const float4*>(qp + off) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  }
  if (has0) load_v(ta_, t0);
  if (has1) load(tb_, t0 + 1);
  if constexpr (I8) {
    // symmetric int8 codes of the column's query row: amax over its D dims
    // (this lane's D / 4 and the three lanes 16 and 32 apart), then codes
    float4 xq[D / 64][4];
    AbsMax am;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xq[ks][e] = qraw[4 * ks + e];
        am.add(xq[ks][e].x); am.add(xq[ks][e].y); am.add(xq[ks][e].z); am.add(xq[ks][e].w);
      }
    float m = am.m, nf = am.nan ? 1.f : 0.f;
    m = fmaxf(m, __shfl_xor(m, 16, kWave));
    m = fmaxf(m, __shfl_xor(m, 32, kWave));
    nf = fmaxf(nf, __shfl_xor(nf, 16, kWave));
    nf = fmaxf(nf, __shfl_xor(nf, 32, kWave));
    AbsMax col;
    col.m = m;
    col.nan = nf != 0.f;
    const float s = col.scale();
    const RowQuant rq(s);
    bool ok = rq.fast;
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        qcode[ks][e] = (int)pack_codes4_fast(xq[ks][e].x, xq[ks][e].y, xq[ks][e].z, xq[ks][e].w, rq, ok);
    if (__any(!ok)) {
#pragma unroll
      for (int ks = 0; ks < D / 64; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          qcode[ks][e] = (int)pack_codes4(xq[ks][e].x, xq[ks][e].y, xq[ks][e].z, xq[ks][e].w, rq);
    }
    sq = s * sl2e;
  } else {
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      const float4 x = qraw[2 * ks], y = qraw[2 * ks + 1];
      float f[8];
      f[0] = x.x * sl2e; f[1] = x.y * sl2e; f[2] = x.z * sl2e; f[3] = x.w * sl2e;
      f[4] = y.x * sl2e; f[5] = y.y * sl2e; f[6] = y.z * sl2e; f[7] = y.w * sl2e;
      qreg[ks] = to_bf16x8(f);
    }
  }

  v4f acc[D / 16];
#pragma unroll
  for (int db = 0; db < D / 16; ++db) acc[db] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  int nf_tile = 0;      // R > 1: the tile whose non-finite values were left out
  uint32_t nf_pos = 0;  // and their positions in it

  // One tile; x is reloaded with tile t + 2 once its operands are consumed.
  // The decode step's new row: the wave whose turn covers its tile rounds it
  // exactly as the append kernel rounds, writes it to the cache at once (its
  // loads overlap the first tiles) and keeps the bf16 row in its LDS merge
  // slot, idle until the end; when it reaches that tile it uses those values
  // in place of what its loads of the tile brought in.  No other wave
  // touches that position.  int8-K: the wave quantises the row as the append
  // kernel does and keeps its codes (as bf16 keeps its rounded row) and its
  // scale s_new.
  uint16_t* row_lds = reinterpret_cast<uint16_t*>(sacc[w]);  // [K row][V row D bf16]
  float s_new = 0.f;
  if (owns_new) {
    const size_t slab_el = ((size_t)b * Hkv + g) * (size_t)C * D;
    uint16_t* vw = reinterpret_cast<uint16_t*>(v_cache) + slab_el;
    const int gv = vbf16_group(p_new), e = vbf16_slot(p_new);
    if constexpr (I8) {
      // lane l: dims 4 l .. 4 l + 3; amax and NaN flag across the wave
      const bool mine = 4 * lane < D;
      const float4 x = nk0;
      AbsMax am;
      am.add(x.x); am.add(x.y); am.add(x.z); am.add(x.w);
      float m = am.m, nf = am.nan ? 1.f : 0.f;
#pragma unroll
      for (int k = 1; k < kWave; k <<= 1) {
        m = fmaxf(m, __shfl_xor(m, k, kWave));
        nf = fmaxf(nf, __shfl_xor(nf, k, kWave));
      }
      AbsMax row;
      row.m = m;
      row.nan = nf != 0.f;
      s_new = row.scale();
      if (mine) {
        // codes of dims 4 l .. + 3: word l % 4 of code vector l / 4 (vectors of a
        // row are 64 vectors apart); the same word index in LDS
        const RowQuant rq(s_new);
        bool ok = rq.fast;
        uint32_t wc = pack_codes4_fast(x.x, x.y, x.z, x.w, rq, ok);
        if (__any(!ok)) wc = pack_codes4(x.x, x.y, x.z, x.w, rq);
        int8_t* kb8 = reinterpret_cast<int8_t*>(k_cache) + slab_el;  // one byte per code
        *reinterpret_cast<uint32_t*>(
            kb8 + (k_vec_index(p_new, 0, D, 16) + (size_t)(lane >> 2) * 64) * 16 + 4 * (lane & 3)) = wc;
        reinterpret_cast<uint32_t*>(row_lds)[lane] = wc;
      }
      if (lane == 0) k_scales[slab_i * C + p_new] = s_new;
    } else {
      uint4* kw = reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_cache) + slab_el);
      if (lane < D / 8) {  // K: one 8-dim vector per lane
        const uint4 o = make_uint4(pack_bf16x2(nk0.x, nk0.y), pack_bf16x2(nk0.z, nk0.w),
                                   pack_bf16x2(nk1.x, nk1.y), pack_bf16x2(nk1.z, nk1.w));
        kw[k_vec_index(p_new, lane, D, 8)] = o;
        reinterpret_cast<uint4*>(row_lds)[lane] = o;
      }
    }
#pragma unroll
    for (int i = 0; i < D / 64; ++i) {  // V: the row's element of each vector
      const int d = lane + 64 * i;
      const uint16_t h = (uint16_t)f32_to_bf16_bits(nv[i]);
      vw[((size_t)gv * D + d) * 8 + e] = h;
      row_lds[D + d] = h;
    }
  }
  auto take_new_row = [&](DecTile<D, I8>& x) {
    const int kp = p_new - kDecTile * t_new;
    // K operand of the new key: 16-byte vector 4 ks + r of the row in LDS (8
    // bf16 values, or 16 int8 codes)
    if (lc == (kp & 15)) {
      const bool hi = (kp >> 4) != 0;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        const uint4 o = reinterpret_cast<const uint4*>(row_lds)[4 * ks + r];
        // 32-bit selects: a branch on the block index would index the
        // register arrays at run time
        x.k[0][ks].x = hi ? x.k[0][ks].x : o.x;
        x.k[0][ks].y = hi ? x.k[0][ks].y : o.y;
        x.k[0][ks].z = hi ? x.k[0][ks].z : o.z;
        x.k[0][ks].w = hi ? x.k[0][ks].w : o.w;
        x.k[1][ks].x = hi ? o.x : x.k[1][ks].x;
        x.k[1][ks].y = hi ? o.y : x.k[1][ks].y;
        x.k[1][ks].z = hi ? o.z : x.k[1][ks].z;
        x.k[1][ks].w = hi ? o.w : x.k[1][ks].w;
      }
    }
    if constexpr (I8) {
      // its scale, in the lanes that hold key kp's scores (keys 16 kb + 4 r + i)
      if (r == ((kp & 15) >> 2)) {
        const bool hi = (kp >> 4) != 0;
        const int i = kp & 3;
        x.sk[0].x = (!hi && i == 0) ? s_new : x.sk[0].x;
        x.sk[0].y = (!hi && i == 1) ? s_new : x.sk[0].y;
        x.sk[0].z = (!hi && i == 2) ? s_new : x.sk[0].z;
        x.sk[0].w = (!hi && i == 3) ? s_new : x.sk[0].w;
        x.sk[1].x = (hi && i == 0) ? s_new : x.sk[1].x;
        x.sk[1].y = (hi && i == 1) ? s_new : x.sk[1].y;
        x.sk[1].z = (hi && i == 2) ? s_new : x.sk[1].z;
        x.sk[1].w = (hi && i == 3) ? s_new : x.sk[1].w;
      }
    }
    if (r == vbf16_group(p_new) - 4 * t_new) {
      const int e = vbf16_slot(p_new);
      // slot e of each register vector: half (e & 1) of 32-bit word e / 2
      const uint32_t sh = (e & 1) * 16, keep = ~(0xffffu << sh);
      const int wd = e >> 1;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        const uint32_t put = (uint32_t)row_lds[D + 16 * db + lc] << sh;
        x.v[db].x = wd == 0 ? (x.v[db].x & keep) | put : x.v[db].x;
        x.v[db].y = wd == 1 ? (x.v[db].y & keep) | put : x.v[db].y;
        x.v[db].z = wd == 2 ? (x.v[db].z & keep) | put : x.v[db].z;
        x.v[db].w = wd == 3 ? (x.v[db].w & keep) | put : x.v[db].w;
      }
    }
  };

  auto tile = [&](DecTile<D, I8>& x, int i) {
    const int t = j0 + i * NW;
    if (owns_new && t == t_new) take_new_row(x);
    v4f sc[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if constexpr (I8) {
        // integer scores, then times the column's and the key's scales
        i32x4 si = {0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          si = __builtin_amdgcn_mfma_i32_16x16x64_i8(__builtin_bit_cast(i32x4, x.k[kb][ks]),
                                                     qcode[ks], si, 0, 0, 0);
        sc[kb][0] = (float)si[0] * (sq * x.sk[kb].x);
        sc[kb][1] = (float)si[1] * (sq * x.sk[kb].y);
        sc[kb][2] = (float)si[2] * (sq * x.sk[kb].z);
        sc[kb][3] = (float)si[3] * (sq * x.sk[kb].w);
      } else {
        sc[kb] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
          sc[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, x.k[kb][ks]),
                                                           qreg[ks], sc[kb], 0, 0, 0);
      }
    }
    // keys past a column's limit get -inf (only tiles reaching past the
    // first limit, ctx - R); positions at or past ctx may hold anything
    const bool tail = kDecTile * t + kDecTile > ctx;
    if (kDecTile * t + kDecTile - 1 > ctx - R) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (kDecTile * t + 16 * kb + 4 * r + i > lim) sc[kb][i] = -INFINITY;
    }
    // column max over the tile: 8 values per lane, then the four row groups
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
    mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
    // online softmax; the reference max moves only when the tile max exceeds
    // it by more than kRescaleSlack (log2 units)
    float alpha = 1.f;
    if (mx > m_run + kRescaleSlack) {
      alpha = fast_exp2(m_run - mx);  // 0 when m_run is -inf
      m_run = mx;
      l_run *= alpha;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;
    uint32_t pk[2][2];  // [kb][pair]: bf16 weights of positions 16 kb + 4 r + 0..3
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = fast_exp2(sc[kb][i] - m_use);
        l_run += p[i];
      }
      pk[kb][0] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)p[0], (__bf16)p[1]});
      pk[kb][1] = __builtin_bit_cast(uint32_t, bf16x2{(__bf16)p[2], (__bf16)p[3]});
    }
    // B operand: slots 0..3 from block 0 of this lane (lower half) or of the
    // lane 32 below (upper half), slots 4..7 from block 0 of the lane 32
    // above (lower half) or block 1 of this lane (upper half)
    uint4 pb;
    {
      const auto x0 = __builtin_amdgcn_permlane32_swap(pk[0][0], pk[1][0], false, false);
      const auto x1 = __builtin_amdgcn_permlane32_swap(pk[0][1], pk[1][1], false, false);
      pb = make_uint4(x0[0], x1[0], x0[1], x1[1]);
    }
    // (the wave's first tile: the sums are still 0, nothing to rescale)
    if (i > 0 && __any(alpha != 1.f)) {
#pragma unroll
      for (int db = 0; db < D / 16; ++db) acc[db] *= alpha;
    }
    if (tail) {
      // zero the values of positions at or past ctx
      uint32_t keep[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        keep[e] = (vbf16_pos(t, r, 2 * e) < ctx ? 0x0000ffffu : 0u) |
                  (vbf16_pos(t, r, 2 * e + 1) < ctx ? 0xffff0000u : 0u);
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        x.v[db].x &= keep[0]; x.v[db].y &= keep[1]; x.v[db].z &= keep[2]; x.v[db].w &= keep[3];
      }
    }
    // Several rows (R > 1): in a tile past the first row's limit the columns
    // share one value product in which a key past a column's limit weighs
    // 0, and 0 * NaN or 0 * inf is NaN.  A non-finite value at such a
    // position (ctx - R < p < ctx) is zeroed for the product; its class and
    // the columns' weights of its position go to this wave's LDS slot (idle
    // until the merge: no new row in this mode), and after the last tile the
    // value reaches only the columns that see it (see class_bf16).  This
    // lane's operand holds dim 16 db + lc of the positions of group r.  The
    // tiles past the first limit all belong to different waves.
    if (ROWS && R > 1 && kDecTile * t + kDecTile - 1 > ctx - R) {
      uint32_t bits = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int p = vbf16_pos(t, r, e);
        const bool inr = p > ctx - R && p < ctx;
#pragma unroll
        for (int db = 0; db < D / 16; ++db) {
          const uint32_t wd = (e >> 1) == 0 ? x.v[db].x : (e >> 1) == 1 ? x.v[db].y
                            : (e >> 1) == 2 ? x.v[db].z : x.v[db].w;
          if (inr && bf16_nonfinite(wd >> (16 * (e & 1)))) bits |= 1u << (p - kDecTile * t);
        }
      }
      const uint32_t nf = wave_or(bits);
      if (nf != 0) {
        nf_tile = t;
        nf_pos = nf;
        uint32_t* tab = reinterpret_cast<uint32_t*>(sacc[w]);  // [32][D / 16] classes
        float* wtab = sacc[w] + kDecTile * (D / 16);           // [32][16] weights
        for (int j = lane; j < kDecTile * (D / 16); j += kWave)
          if ((nf >> (j / (D / 16))) & 1u) tab[j] = 0u;
        wave_lds_sync();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int p = vbf16_pos(t, r, e);
          const bool inr = p > ctx - R && p < ctx;
          const uint32_t sh = 16 * (e & 1);
#pragma unroll
          for (int db = 0; db < D / 16; ++db) {
            uint32_t wd = (e >> 1) == 0 ? x.v[db].x : (e >> 1) == 1 ? x.v[db].y
                        : (e >> 1) == 2 ? x.v[db].z : x.v[db].w;
            if (inr && bf16_nonfinite(wd >> sh)) {
              atomicOr(tab + (p - kDecTile * t) * (D / 16) + db, class_bf16(wd >> sh) << (2 * lc));
              wd &= ~(0xffffu << sh);
              if ((e >> 1) == 0) x.v[db].x = wd;
              else if ((e >> 1) == 1) x.v[db].y = wd;
              else if ((e >> 1) == 2) x.v[db].z = wd;
              else x.v[db].w = wd;
            }
          }
        }
        // weights of this lane's positions 16 kb + 4 r + i (column lc)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int k = 16 * kb + 4 * r + i;
            const uint32_t pw = pk[kb][i >> 1];
            if ((nf >> k) & 1u)
              wtab[k * kDecCols + lc] = __uint_as_float((i & 1) ? (pw & 0xffff0000u) : (pw << 16));
          }
        wave_lds_sync();
      }
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          __builtin_bit_cast(bf16x8, x.v[db]), __builtin_bit_cast(bf16x8, pb), acc[db], 0, 0, 0);
    if (i + 2 < t1) load(x, i + 2);
  };
  for (int t = t0; t < t1; t += 2) {
    tile(ta_, t);
    if (t + 1 < t1) tile(tb_, t + 1);
  }
  // values left out of a tile's shared product (R > 1, rare): into the
  // columns that see them; lane (lc, r) holds dims 16 db + 4 r + 0..3
  if (ROWS && nf_pos != 0) {
    const uint32_t* tab = reinterpret_cast<const uint32_t*>(sacc[w]);
    const float* wtab = sacc[w] + kDecTile * (D / 16);
    uint32_t cls[D / 64];  // dims 16 db + 4 r + i at bits 8 (db % 4) + 2 i of cls[db / 4]
#pragma unroll
    for (int j = 0; j < D / 64; ++j) cls[j] = 0u;
    uint32_t m = nf_pos;
    while (m != 0) {
      const int k = __builtin_ctz(m);
      m &= m - 1;
      if (!hv || kDecTile * nf_tile + k > lim) continue;
      const bool zero_w = wtab[k * kDecCols + lc] == 0.f;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        uint32_t byte = (tab[k * (D / 16) + db] >> (8 * r)) & 0xffu;
        if (zero_w) byte = all_nan(byte);
        cls[db >> 2] |= byte << (8 * (db & 3));
      }
    }
#pragma unroll
    for (int db = 0; db < D / 16; ++db) apply_classes<4>(cls[db >> 2] >> (8 * (db & 3)), acc[db], 0);
    wave_lds_sync();  // the slot takes the accumulators next
  }

  // ---- merge the four waves
  float lt = l_run;
  lt += __shfl_xor(lt, 16, kWave);
  lt += __shfl_xor(lt, 32, kWave);
  if (lc < hpw) {
    float* o = sacc[w] + lc * D;
    // lane holds dims 16 db + 4 r + 0..3
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<float4*>(o + 16 * db + 4 * r) =
          make_float4(acc[db][0], acc[db][1], acc[db][2], acc[db][3]);
    if (r == 0) {
      wm[w][lc] = m_run;
      wl[w][lc] = lt;
    }
  }
  __syncthreads();
  const int gq = b * (Hkv * HG) + gh;  // partial slot of (b, g, hg)
  for (int i = tid; i < hpw * D / 4; i += 256) {
    const int h = i / (D / 4), d = 4 * (i % (D / 4));
    const int ph = hg * hpw + h;  // row ph / G, head g G + ph % G
    if (ph >= R * G) continue;
    float M = -INFINITY;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) M = fmaxf(M, wm[ww][h]);
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    float l = 0.f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float f = wm[ww][h] == -INFINITY ? 0.f : fast_exp2(wm[ww][h] - M);
      const float4 x = *reinterpret_cast<const float4*>(sacc[ww] + h * D + d);
      a.x += f * x.x; a.y += f * x.y; a.z += f * x.z; a.w += f * x.w;
      l += f * wl[ww][h];
    }
    if (S == 1) {
      const float inv = 1.f / l;
      *reinterpret_cast<float4*>(out + (((size_t)b * R + (ROWS ? ph / G : 0)) * Hq + g * G +
                                        (ROWS ? ph % G : ph)) * D + d) =
          make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    } else {
      *reinterpret_cast<float4*>(part + (((size_t)gq * S + split) * hpw + h) * D + d) = a;
      if (d == 0) {
        part_ml[(((size_t)gq * hpw + h) * S + split) * 2] = M;
        part_ml[(((size_t)gq * hpw + h) * S + split) * 2 + 1] = l;
      }
    }
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
                  float* out, float* part, const float* k_new, const float* v_new,
                  const CtxArg& ca, int b0, const Shape& s, int HG, int S, float sl2e) {
  float* part_ml = part + (size_t)s.batch * s.num_kv_heads * HG * S * HPW * D;
  hipLaunchKernelGGL((decode_split_kernel<D, HPW, BF16>), grid, dim3(256), 0, st, q, kc, vc, out,
                     part, part_ml, k_new, v_new, ca, b0, s.num_q_heads, s.num_kv_heads, HG,
                     s.capacity, S, sl2e);
}

template <int D, bool BF16>
void dispatch_hpw(int hpw, dim3 grid, hipStream_t st, const float* q, const void* kc,
                  const void* vc, float* out, float* part, const float* k_new, const float* v_new,
                  const CtxArg& ca, int b0, const Shape& s, int HG, int S, float sl2e) {
  switch (hpw) {
    case 8: launch_split<D, 8, BF16>(grid, st, q, kc, vc, out, part, k_new, v_new, ca, b0, s, HG, S, sl2e); break;
    case 4: launch_split<D, 4, BF16>(grid, st, q, kc, vc, out, part, k_new, v_new, ca, b0, s, HG, S, sl2e); break;
    case 2: launch_split<D, 2, BF16>(grid, st, q, kc, vc, out, part, k_new, v_new, ca, b0, s, HG, S, sl2e); break;
    default: launch_split<D, 1, BF16>(grid, st, q, kc, vc, out, part, k_new, v_new, ca, b0, s, HG, S, sl2e); break;
  }
}

// 1-D grid of the MFMA kernel: one workgroup per item, padded to whole
// rounds of the 8 XCDs when head groups are remapped
dim3 mfma_grid(int nb, int Hkv, int HG, int S) {
  if (HG == 1) return dim3((unsigned)S, (unsigned)Hkv, (unsigned)nb);
  const long long n = (long long)nb * Hkv * HG * S;
  return dim3((unsigned)(8 * ((n + 7) / 8)));
}

template <int D>
void launch_merge(int hpw, dim3 grid, hipStream_t st, const float* part, float* out, int b0,
                  const Shape& s, int HG, int S, int R = 1) {
  const float* ml = part + (size_t)s.batch * s.num_kv_heads * HG * S * hpw * D;
  auto go = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, st, part, ml, out, b0, s.num_q_heads,
                       s.num_kv_heads, HG, hpw, S, R);
  };
  // batches of 8 splits loaded at once: ceil(S / 8), rounded up to 1, 2, 4
  // or a multiple of 4 (at most 3 batches loaded for nothing)
  const int nb = (S + 7) / 8;
  if (nb <= 1) go(decode_merge_kernel<D, 1>);
  else if (nb <= 2) go(decode_merge_kernel<D, 2>);
  else if (nb <= 4) go(decode_merge_kernel<D, 4>);
  else if (nb <= 8) go(decode_merge_kernel<D, 8>);
  else if (nb <= 12) go(decode_merge_kernel<D, 12>);
  else if (nb <= 16) go(decode_merge_kernel<D, 16>);
  else if (nb <= 20) go(decode_merge_kernel<D, 20>);
  else if (nb <= 24) go(decode_merge_kernel<D, 24>);
  else if (nb <= 28) go(decode_merge_kernel<D, 28>);
  else go(decode_merge_kernel<D, kMergeEarly>);
}

}  // namespace

// f32 caches (VALU kernel): heads per workgroup and splits for a context of
// `units` 16-position units.  A wave's work per unit grows with the heads it
// serves, and short steps are bound by that chain of one wave, not by bytes:
// while the whole step is small (every slab's units together at most
// kF32FewUnits, e.g. one session at 4097 keys) a workgroup serves a quarter
// of the heads and two units, so four times as many waves each do an eighth
// of the work (4097 keys: 12.5 us against 17.4 us with all 8 heads and four
// units); up to kF32MidUnits, half the heads (one session at 16K: 20.7
// against 22.2 us).  Past that the step streams the cache, and every head
// group would read it again, so a workgroup serves all heads (4 sessions at
// 64K: 108 us against 136 us with half).
constexpr long long kF32FewUnits = 512, kF32MidUnits = 2048;

struct F32Plan {
  int hpw;
  long long S;
};

static F32Plan plan_f32(const Shape& s, int units) {
  const int G = s.num_q_heads / s.num_kv_heads;
  const int h0 = heads_per_wg(G);
  const long long work = (long long)s.batch * s.num_kv_heads * units;
  int hpw = h0, upw = kWaves;
  if (work <= kF32FewUnits) {
    hpw = h0 >= 4 ? h0 / 4 : 1;
    upw = 2;
  } else if (work <= kF32MidUnits) {
    hpw = h0 >= 2 ? h0 / 2 : 1;
  }
  const long long slabs = (long long)s.batch * s.num_kv_heads * (G / hpw);
  long long S = (kTargetWgs + slabs - 1) / slabs;
  // at most about one unit per active wave: with fewer splits some wave gets
  // a second unit and runs two dependent load-then-compute rounds
  const long long by_units = (units + upw - 1) / upw;
  if (S > by_units) S = by_units;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  return {hpw, S};
}

// Partial bytes of a split plan: acc [slab][S][HPW][D], then (m, l)
// [slab][HPW][S][2]; none with one split.
static size_t part_bytes(const Shape& s, long long slabs, int hpw, long long S) {
  return S == 1 ? 0 : (size_t)slabs * S * hpw * (s.head_dim + 2) * sizeof(float);
}

DecodePlan plan_decode(const Shape& s, int max_ctx) {
  DecodePlan p;
  const int G = s.num_q_heads / s.num_kv_heads;
  if (s.kv_dtype != kF32) {
    // MFMA path (bf16 and int8-K caches): up to 16 heads share a workgroup's columns; one round of
    // 256 workgroups (one per CU: a wave's operand registers fill its SIMD),
    // at least one tile per wave
    int hg = 1;
    while (G / hg > kDecCols || G % hg != 0) ++hg;
    p.head_groups = hg;
    p.heads_per_wg = G / hg;
    const long long slabs = (long long)s.batch * s.num_kv_heads * hg;
    const long long tiles = (max_ctx + kDecTile - 1) / kDecTile;
    long long S = 256 / slabs;  // a 257th workgroup would start a second round
    const long long by_tiles = (tiles + kWaves - 1) / kWaves;
    if (S > by_tiles) S = by_tiles;
    if (S > kMaxSplits) S = kMaxSplits;
    if (S < 1) S = 1;
    p.splits = (int)S;
    // S grows with the context, so this also covers every shorter context
    p.workspace_bytes = part_bytes(s, slabs, p.heads_per_wg, S);
    return p;
  }
  const int units = units_for(max_ctx);
  const F32Plan f = plan_f32(s, units);
  p.heads_per_wg = f.hpw;
  p.head_groups = G / f.hpw;
  p.splits = (int)f.S;
  // The workspace bound covers every context up to max_ctx (a caller sizes
  // it once, at the longest): within one regime S grows with the context,
  // but a step into the next regime can lower it, so the last context of
  // each shorter regime is taken too.
  const long long per = (long long)s.batch * s.num_kv_heads;
  size_t ws = 0;
  for (const long long lim : {kF32FewUnits, kF32MidUnits}) {
    const long long u = lim / per;  // the last unit count of that regime
    if (u < 1 || u >= units) continue;
    const F32Plan e = plan_f32(s, (int)u);
    const size_t b = part_bytes(s, per * (G / e.hpw), e.hpw, e.S);
    if (b > ws) ws = b;
  }
  const size_t own = part_bytes(s, per * p.head_groups, f.hpw, f.S);
  p.workspace_bytes = own > ws ? own : ws;
  return p;
}

DecodePlan plan_rows(const Shape& s, int R, int ctx) {
  DecodePlan p;
  const int G = s.num_q_heads / s.num_kv_heads;
  const int pairs = R * G;
  p.head_groups = (pairs + kDecCols - 1) / kDecCols;
  p.heads_per_wg = (pairs + p.head_groups - 1) / p.head_groups;
  const long long slabs = (long long)s.batch * s.num_kv_heads * p.head_groups;
  const long long tiles = (ctx + kDecTile - 1) / kDecTile;
  long long S = 256 / slabs;  // one round: one workgroup per CU
  const long long by_tiles = (tiles + kWaves - 1) / kWaves;
  if (S > by_tiles) S = by_tiles;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S < 1) S = 1;
  p.splits = (int)S;
  p.workspace_bytes = p.splits == 1 ? 0
      : (size_t)slabs * p.splits * p.heads_per_wg * (s.head_dim + 2) * sizeof(float);
  return p;
}

hipError_t launch_rows(const Shape& s, const DecodePlan& p, const float* q, const void* k_cache,
                       const void* v_cache, float* out, int start, int R, float scale,
                       void* workspace, hipStream_t stream) {
  if (s.kv_dtype == kF32) return hipErrorInvalidValue;
  const float sl2e = scale * kLog2e;
  const int HG = p.head_groups, S = p.splits, hpw = p.heads_per_wg;
  float* part = reinterpret_cast<float*>(workspace);
  void* kc = const_cast<void*>(k_cache);  // read only: the kernel writes only new rows, and none are given
  void* vc = const_cast<void*>(v_cache);
  for (int b0 = 0; b0 < s.batch; b0 += kMaxDecodeBatchPerLaunch) {
    const int nb = s.batch - b0 < kMaxDecodeBatchPerLaunch ? s.batch - b0 : kMaxDecodeBatchPerLaunch;
    CtxArg ca;
    for (int i = 0; i < kMaxDecodeBatchPerLaunch; ++i) ca.ctx[i] = start + R;
    switch (s.head_dim) {
#define KA_D(DD)                                                                               \
  case DD:                                                                                     \
    if (s.kv_dtype == kI8K)                                                                    \
      hipLaunchKernelGGL((decode_mfma_kernel<DD, true, true>), mfma_grid(nb, s.num_kv_heads, HG, S), \
                         dim3(256), 0, stream, q, kc, vc, out, part,                           \
                         part + (size_t)s.batch * s.num_kv_heads * HG * S * hpw * DD, nullptr, \
                         nullptr, k_scale_array(s, kc), ca, b0, nb, s.num_q_heads,             \
                         s.num_kv_heads, HG, hpw, s.capacity, S, sl2e, R);                     \
    else                                                                                       \
      hipLaunchKernelGGL((decode_mfma_kernel<DD, false, true>), mfma_grid(nb, s.num_kv_heads, HG, S),\
                         dim3(256), 0, stream, q, kc, vc, out, part,                           \
                         part + (size_t)s.batch * s.num_kv_heads * HG * S * hpw * DD, nullptr, \
                         nullptr, nullptr, ca, b0, nb, s.num_q_heads, s.num_kv_heads, HG, hpw, \
                         s.capacity, S, sl2e, R);                                              \
    if (S > 1) launch_merge<DD>(hpw, dim3(hpw * (DD / 32), s.num_kv_heads * HG, nb), stream,  \
                                part, out, b0, s, HG, S, R);                                   \
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

hipError_t launch_decode(const Shape& s, const DecodePlan& p, const float* q, void* k_cache,
                         void* v_cache, float* out, const int32_t* ctx_host, float scale,
                         void* workspace, hipStream_t stream, const float* k_new,
                         const float* v_new) {
  const bool bf16 = s.kv_dtype == kBF16, i8 = s.kv_dtype == kI8K;
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
    if (bf16)                                                                                  \
      hipLaunchKernelGGL((decode_mfma_kernel<DD, false, false>), mfma_grid(nb, s.num_kv_heads, HG, S),\
                         dim3(256), 0, stream, q, k_cache, v_cache, out, part,                 \
                         part + (size_t)s.batch * s.num_kv_heads * HG * S * p.heads_per_wg * DD, \
                         k_new, v_new, nullptr, ca, b0, nb, s.num_q_heads, s.num_kv_heads, HG, \
                         p.heads_per_wg,                                                       \
                         s.capacity, S, sl2e, 1);                                              \
    else if (i8)                                                                               \
      hipLaunchKernelGGL((decode_mfma_kernel<DD, true, false>), mfma_grid(nb, s.num_kv_heads, HG, S), \
                         dim3(256), 0, stream, q, k_cache, v_cache, out, part,                 \
                         part + (size_t)s.batch * s.num_kv_heads * HG * S * p.heads_per_wg * DD, \
                         k_new, v_new, k_scale_array(s, k_cache), ca, b0, nb,                  \
                         s.num_q_heads, s.num_kv_heads, HG, p.heads_per_wg, s.capacity, S,     \
                         sl2e, 1);                                                             \
    else dispatch_hpw<DD, false>(p.heads_per_wg, grid, stream, q, k_cache, v_cache, out, part, \
                                 k_new, v_new, ca, b0, s, HG, S, sl2e);                        \
    if (S > 1) launch_merge<DD>(p.heads_per_wg,                                               \
                                dim3(p.heads_per_wg * (DD / 32), s.num_kv_heads * HG, nb),     \
                                stream, part, out, b0, s, HG, S);                              \
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
