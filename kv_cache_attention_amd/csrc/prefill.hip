// Chunked prefill on MFMA: rows start .. start+R-1 attend causally to the
// cache of their session.
//
// Tiling.  One workgroup (4 waves) owns an M-tile of 128 (row, query head)
// pairs of one KV head -- for 8 heads per KV head that is 16 consecutive rows
// x 8 heads -- and a range of 64-position key tiles (one split of the causal
// key range).  Each K / V tile is staged once in LDS and read by all four
// waves, so every K / V row is fetched once per M-tile, i.e. once per 128 / G
// chunk rows and shared by every query head of the group.  Each wave owns 32
// of the 128 M columns.
//
// Products.  Scores are computed transposed, S^T = K . Q^T (M = 16 keys,
// N = 16 (row, head) pairs), and values as O^T = V^T . P^T (M = 16 dims).  In
// the MFMA accumulator layout a lane then holds one (row, head) column and 4
// keys / dims, so the running max, the running sum and the rescale of the
// accumulator are lane-local, and the exponentiated S^T registers are
// already the B operand of the value product: the V layout groups positions
// {4s..4s+3, 16+4s..16+4s+3} of a 32-block exactly as a lane group holds
// them.  bf16 caches use v_mfma_f32_16x16x32_bf16 with Q and P rounded to
// bf16 and f32 accumulation; f32 caches use v_mfma_f32_16x16x4_f32.
//
// Softmax.  Online (flash-style) in f32, log2 domain.  Only tiles that cross
// a row's causal limit are masked; tiles above every row's limit are not
// visited.  Positions at or beyond start + R are zeroed in LDS so that
// whatever the cache holds there cannot reach a result.
#include <type_traits>

#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

namespace {

constexpr int kMTile = 128;
constexpr int kNTile = 64;
constexpr int kTargetWgs = 512;
constexpr int kMaxSplits = 64;

typedef __attribute__((ext_vector_type(4))) float v4f;

template <int D, bool BF16>
struct PrefillCfg {
  static constexpr int E = Elem<BF16>::E;
  static constexpr int KVEC = D / E * kNTile;            // 16-byte vectors per K tile
  static constexpr int VVEC = kNTile / E * D;            // 16-byte vectors per V tile
  static constexpr int TILE_BYTES = KVEC * 16;           // same for V
  static constexpr int NDB = D / 16;                     // 16-dim output blocks
};

__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = __builtin_bit_cast(__bf16, (uint16_t)f32_to_bf16_bits(f[j]));
  return r;
}

// partial row layout in the workspace: acc[D], m, l, 2 pad floats
template <int D> constexpr int part_stride() { return D + 4; }

template <int D, bool BF16>
__global__ __launch_bounds__(256) void prefill_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    int Hq, int Hkv, int C, int start, int R, int m_tiles, int S, float sl2e) {
  using Cfg = PrefillCfg<D, BF16>;
  constexpr int E = Cfg::E;
  constexpr int NDB = Cfg::NDB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint4* k_lds = reinterpret_cast<uint4*>(smem);
  uint4* v_lds = reinterpret_cast<uint4*>(smem + Cfg::TILE_BYTES);

  // ---- block -> (m-tile, split), XCD-aware: blocks x, x+8, x+16, ... land on
  // one XCD; give them the same key range so its L2 serves all of them.
  const int x = blockIdx.x;
  int mt, split;
  if (S >= 8 && S % 8 == 0) {
    const int spx = S / 8, xcd = x & 7, j = x >> 3;
    split = xcd * spx + j % spx;
    mt = j / spx;
  } else {
    mt = x / S;
    split = x % S;
  }
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int M_total = R * G;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int lr = lane & 15, lg = lane >> 4;

  const int m_base = mt * kMTile;
  const int row_lo = m_base / G;
  const int row_hi = min(R - 1, (m_base + kMTile - 1) / G);
  const int nkt = (start + row_hi) / kNTile + 1;
  const int kt0 = (int)((long long)split * nkt / S);
  const int kt1 = (int)((long long)(split + 1) * nkt / S);
  const int kend = start + R;  // first position not appended by this chunk

  // this lane's two M columns (mb = 0, 1)
  int m_col[2], row_col[2];
  bool valid_col[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    m_col[mb] = m_base + w * 32 + mb * 16 + lr;
    valid_col[mb] = m_col[mb] < M_total;
    row_col[mb] = valid_col[mb] ? m_col[mb] / G : 0;
  }
  auto q_row_ptr = [&](int mb) -> const float* {
    const int m = m_col[mb];
    const int row = m / G, hh = m % G;
    return q + (((size_t)b * R + row) * Hq + g * G + hh) * D;
  };

  // ---- stationary Q^T operand in registers
  constexpr int NQ = BF16 ? D / 32 : D / 16;
  typename std::conditional<BF16, bf16x8, v4f>::type qreg[2][NQ];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const float* qp = q_row_ptr(mb);
#pragma unroll
    for (int ks = 0; ks < NQ; ++ks) {
      if constexpr (BF16) {
        float f[8];
        if (valid_col[mb]) {
          const float4 a = *reinterpret_cast<const float4*>(qp + 32 * ks + 8 * lg);
          const float4 c = *reinterpret_cast<const float4*>(qp + 32 * ks + 8 * lg + 4);
          f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
          f[4] = c.x; f[5] = c.y; f[6] = c.z; f[7] = c.w;
        } else {
#pragma unroll
          for (int j = 0; j < 8; ++j) f[j] = 0.f;
        }
        qreg[mb][ks] = to_bf16x8(f);
      } else {
        v4f a = {0.f, 0.f, 0.f, 0.f};
        if (valid_col[mb]) {
          const float4 t = *reinterpret_cast<const float4*>(qp + 16 * ks + 4 * lg);
          a[0] = t.x; a[1] = t.y; a[2] = t.z; a[3] = t.w;
        }
        qreg[mb][ks] = a;
      }
    }
  }

  v4f acc_o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};

  const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;  // elements
  const unsigned char* kbase = reinterpret_cast<const unsigned char*>(k_cache) + slab * (BF16 ? 2 : 4);
  const unsigned char* vbase = reinterpret_cast<const unsigned char*>(v_cache) + slab * (BF16 ? 2 : 4);

  for (int kt = kt0; kt < kt1; ++kt) {
    // ---- stage the K and V tiles (both contiguous in the cache)
    const uint4* ksrc = reinterpret_cast<const uint4*>(kbase + (size_t)kt * Cfg::TILE_BYTES);
    const uint4* vsrc = reinterpret_cast<const uint4*>(vbase + (size_t)kt * Cfg::TILE_BYTES);
    const bool last = (kt + 1) * kNTile > kend;
    __syncthreads();  // previous tile fully consumed
#pragma unroll 4
    for (int i = tid; i < Cfg::KVEC; i += 256) k_lds[i] = ksrc[i];
#pragma unroll 4
    for (int i = tid; i < Cfg::VVEC; i += 256) {
      uint4 v = vsrc[i];
      if (last) {
        // vector i of the tile: group i / D holds E positions
        const int gi = i / D;
        uint32_t keep[4];
        if constexpr (BF16) {
          const int blk = kt * 2 + (gi >> 2), sg = gi & 3;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            keep[e] = (vbf16_pos(blk, sg, 2 * e) < kend ? 0x0000ffffu : 0u) |
                      (vbf16_pos(blk, sg, 2 * e + 1) < kend ? 0xffff0000u : 0u);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) keep[e] = (kt * kNTile + gi * 4 + e) < kend ? ~0u : 0u;
        }
        v.x &= keep[0]; v.y &= keep[1]; v.z &= keep[2]; v.w &= keep[3];
      }
      v_lds[i] = v;
    }
    __syncthreads();

    // ---- S^T = K . Q^T for 4 key blocks x 2 column blocks
    v4f sacc[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) sacc[kb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 a = k_lds[(4 * ks + lg) * 64 + 16 * kb + lr];
          const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            sacc[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, qreg[mb][ks], sacc[kb][mb], 0, 0, 0);
        }
      }
    } else {
#pragma unroll
      for (int c4 = 0; c4 < D / 16; ++c4) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 a = k_lds[(4 * c4 + lg) * 64 + 16 * kb + lr];
          const float av[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                               __uint_as_float(a.w)};
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              sacc[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], qreg[mb][c4][t], sacc[kb][mb], 0, 0, 0);
        }
      }
    }

    // ---- causal mask (only tiles that cross some row's limit), online softmax
    const bool diag = kt * kNTile + kNTile - 1 > start + row_lo;
    float alpha[2];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int lim = start + row_col[mb];
      // scores to the log2 domain first, so the row's largest term is
      // exactly exp2(0) = 1
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float sv = sacc[kb][mb][i] * sl2e;
          if (diag) {
            const int key = kt * kNTile + 16 * kb + 4 * lg + i;
            if (key > lim || !valid_col[mb]) sv = -INFINITY;
          }
          sacc[kb][mb][i] = sv;
          mx = fmaxf(mx, sv);
        }
      mx = fmaxf(mx, xor_shfl(mx, 16));
      mx = fmaxf(mx, xor_shfl(mx, 32));
      const float m_new = fmaxf(m_run[mb], mx);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      alpha[mb] = fast_exp2(m_run[mb] - m_use);
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(sacc[kb][mb][i] - m_use);
          sacc[kb][mb][i] = pv;
          ls += pv;
        }
      l_run[mb] = l_run[mb] * alpha[mb] + ls;
      m_run[mb] = m_new;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] *= alpha[mb];

    // ---- O^T += V^T . P^T
    if constexpr (BF16) {
      bf16x8 pb[2][2];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          float f[8];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f[i] = sacc[2 * k2][mb][i];
            f[4 + i] = sacc[2 * k2 + 1][mb][i];
          }
          pb[mb][k2] = to_bf16x8(f);
        }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int k2 = 0; k2 < 2; ++k2) {
          const uint4 a = v_lds[(k2 * 4 + lg) * D + 16 * db + lr];
          const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
            acc_o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, pb[mb][k2], acc_o[db][mb], 0, 0, 0);
        }
    } else {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const uint4 a = v_lds[(4 * kb + lg) * D + 16 * db + lr];
          const float av[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                               __uint_as_float(a.w)};
#pragma unroll
          for (int mb = 0; mb < 2; ++mb)
#pragma unroll
            for (int t = 0; t < 4; ++t)
              acc_o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[t], sacc[kb][mb][t], acc_o[db][mb], 0, 0, 0);
        }
    }
  }

  // ---- epilogue: lane holds O^T[16 db + 4 lg + i][column]
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float lt = l_run[mb];
    lt += xor_shfl(lt, 16);
    lt += xor_shfl(lt, 32);
    if (!valid_col[mb]) continue;
    if (S == 1) {
      const int m = m_col[mb];
      const int row = m / G, hh = m % G;
      float* op = out + (((size_t)b * R + row) * Hq + g * G + hh) * D;
      const float inv = 1.f / lt;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc_o[db][mb] * inv;
        *reinterpret_cast<float4*>(op + 16 * db + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      const size_t slot = ((((size_t)b * Hkv + g) * m_tiles + mt) * S + split) * kMTile +
                          (m_col[mb] - m_base);
      float* pp = part + slot * part_stride<D>();
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc_o[db][mb];
        *reinterpret_cast<float4*>(pp + 16 * db + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (lg == 0) {
        pp[D] = m_run[mb];
        pp[D + 1] = lt;
      }
    }
  }
}

// Combines the S split partials of every column of one M-tile, in split order.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    const float* __restrict__ part, float* __restrict__ out, int Hq, int Hkv, int R,
    int m_tiles, int S) {
  __shared__ float wgt[kMTile * kMaxSplits];
  __shared__ float inv_l[kMTile];
  const int mt = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int M_total = R * G;
  const int tid = threadIdx.x;
  constexpr int PS = part_stride<D>();
  const float* pb = part + (((size_t)b * Hkv + g) * m_tiles + mt) * (size_t)S * kMTile * PS;
  for (int c = tid; c < kMTile; c += 256) {
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, pb[((size_t)s * kMTile + c) * PS + D]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float* e = pb + ((size_t)s * kMTile + c) * PS;
      const float f = e[D] == -INFINITY ? 0.f : fast_exp2(e[D] - M);
      wgt[c * kMaxSplits + s] = f;
      L += f * e[D + 1];
    }
    inv_l[c] = 1.f / L;
  }
  __syncthreads();
  constexpr int NV = D / 4;
  for (int i = tid; i < kMTile * NV; i += 256) {
    const int c = i / NV, dv = i % NV;
    const int m = mt * kMTile + c;
    if (m >= M_total) continue;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < S; ++s) {
      const float f = wgt[c * kMaxSplits + s];
      const float4 v = *reinterpret_cast<const float4*>(pb + ((size_t)s * kMTile + c) * PS + 4 * dv);
      a.x += f * v.x; a.y += f * v.y; a.z += f * v.z; a.w += f * v.w;
    }
    const float il = inv_l[c];
    const int row = m / G, hh = m % G;
    float* op = out + (((size_t)b * R + row) * Hq + g * G + hh) * D;
    *reinterpret_cast<float4*>(op + 4 * dv) = make_float4(a.x * il, a.y * il, a.z * il, a.w * il);
  }
}

int choose_splits(const Shape& s, int m_tiles, int nkt) {
  const long long wgs = (long long)s.batch * s.num_kv_heads * m_tiles;
  long long S = (kTargetWgs + wgs / 2) / wgs;
  if (S >= 8) S = S / 8 * 8;
  if (S > kMaxSplits) S = kMaxSplits;
  if (S > nkt) S = nkt;
  if (S > 8 && S % 8) S = S / 8 * 8;
  if (S < 1) S = 1;
  return (int)S;
}

template <int D, bool BF16>
hipError_t launch_t(const Shape& s, const PrefillPlan& p, const float* q, const void* kc,
                    const void* vc, float* out, int start, int R, float scale, void* ws,
                    hipStream_t st) {
  using Cfg = PrefillCfg<D, BF16>;
  const size_t lds = 2 * Cfg::TILE_BYTES;
  auto kern = prefill_kernel<D, BF16>;
  hipError_t e = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     (int)lds);
  if (e != hipSuccess) return e;
  dim3 grid(p.m_tiles * p.splits, s.num_kv_heads, s.batch);
  hipLaunchKernelGGL(kern, grid, dim3(256), lds, st, q, kc, vc, out,
                     reinterpret_cast<float*>(ws), s.num_q_heads, s.num_kv_heads, s.capacity,
                     start, R, p.m_tiles, p.splits, scale * kLog2e);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    hipLaunchKernelGGL(prefill_merge_kernel<D>, dim3(p.m_tiles, s.num_kv_heads, s.batch),
                       dim3(256), 0, st, reinterpret_cast<const float*>(ws), out,
                       s.num_q_heads, s.num_kv_heads, R, p.m_tiles, p.splits);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

PrefillPlan plan_prefill(const Shape& s, int start, int R) {
  PrefillPlan p;
  const int G = s.num_q_heads / s.num_kv_heads;
  const long long M = (long long)R * G;
  p.m_tiles = (int)((M + kMTile - 1) / kMTile);
  const int nkt = (start + R - 1) / kNTile + 1;
  p.splits = choose_splits(s, p.m_tiles, nkt);
  p.workspace_bytes = p.splits == 1 ? 0
      : (size_t)s.batch * s.num_kv_heads * p.m_tiles * p.splits * kMTile *
            (size_t)(s.head_dim + 4) * sizeof(float);
  return p;
}

size_t prefill_workspace_bound(const Shape& s, int max_rows) {
  if (max_rows <= 0) return 0;
  const int G = s.num_q_heads / s.num_kv_heads;
  const int mt_max = (int)(((long long)max_rows * G + kMTile - 1) / kMTile);
  size_t best = 0;
  for (int mt = 1; mt <= mt_max; ++mt) {
    const int S = choose_splits(s, mt, 1 << 30);
    if (S == 1) continue;
    const size_t bytes = (size_t)s.batch * s.num_kv_heads * mt * S * kMTile *
                         (size_t)(s.head_dim + 4) * sizeof(float);
    if (bytes > best) best = bytes;
  }
  return best;
}

hipError_t launch_prefill(const Shape& s, const PrefillPlan& p, const float* q,
                          const void* k_cache, const void* v_cache, float* out, int start, int R,
                          float scale, void* workspace, hipStream_t stream) {
  const bool bf16 = s.kv_dtype == 1;
  switch (s.head_dim) {
    case 64: return bf16 ? launch_t<64, true>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream)
                         : launch_t<64, false>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream);
    case 128: return bf16 ? launch_t<128, true>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream)
                          : launch_t<128, false>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream);
    case 256: return bf16 ? launch_t<256, true>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream)
                          : launch_t<256, false>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ka
