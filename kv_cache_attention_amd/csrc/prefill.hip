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
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay below 256

typedef __attribute__((ext_vector_type(4))) float v4f;

template <int D, bool BF16>
struct PrefillCfg {
  static constexpr int E = Elem<BF16>::E;
  static constexpr int KVEC = D / E * kNTile;            // 16-byte vectors per K tile
  static constexpr int VVEC = kNTile / E * D;            // 16-byte vectors per V tile
  static constexpr int TILE_BYTES = KVEC * 16;           // same for V
  static constexpr int NDB = D / 16;                     // 16-dim output blocks
  // double-buffered K+V tiles when two stages fit in the 160 KiB of LDS
  static constexpr int STAGES = 4 * TILE_BYTES <= 160 * 1024 ? 2 : 1;
  static constexpr int LDS_BYTES = STAGES * 2 * TILE_BYTES;
};

// Asynchronous copy of one K tile and one V tile (each TILE_BYTES contiguous
// bytes in the cache) into LDS with global_load_lds: every wave instruction
// moves 1 KiB, lane l's 16 bytes landing at the wave's LDS base + 16 l.
template <int TILE_BYTES>
__device__ __forceinline__ void stage_tiles(const unsigned char* ksrc, const unsigned char* vsrc,
                                            unsigned char* kdst, unsigned char* vdst, int w,
                                            int lane) {
  constexpr int PER_THREAD = TILE_BYTES / (256 * 16);
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int off = (i * 256 + w * 64) * 16;
    __builtin_amdgcn_global_load_lds(
        (const void*)(ksrc + off + lane * 16),
        (__attribute__((address_space(3))) void*)(kdst + off), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(
        (const void*)(vsrc + off + lane * 16),
        (__attribute__((address_space(3))) void*)(vdst + off), 16, 0, 0);
  }
}

// s_waitcnt vmcnt(0) through the builtin (not inline asm), so the compiler's
// own wait tracking sees it.  gfx9 encoding: vmcnt 0, expcnt 7, lgkmcnt 15.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// MFMA operands (Q, P) are rounded with the hardware converter
// (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ bf16x8 to_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int j = 0; j < 8; ++j) r[j] = (__bf16)f[j];
  return r;
}


template <int D, bool BF16>
__global__ __launch_bounds__(256) void prefill_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    float* __restrict__ part_ml, int Hq, int Hkv, int C, int start, int R, int m_tiles, int S,
    float sl2e) {
  using Cfg = PrefillCfg<D, BF16>;
  constexpr int E = Cfg::E;
  constexpr int NDB = Cfg::NDB;
  constexpr int STAGES = Cfg::STAGES;
  // Two distinct LDS objects (one per stage): the compiler can then tell that
  // the asynchronous copy into one stage does not alias reads of the other,
  // and issues no wait for it before the compute.
  __shared__ __attribute__((aligned(16))) unsigned char stage0[2 * Cfg::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char stage1[STAGES == 2 ? 2 * Cfg::TILE_BYTES : 16];

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
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, kept in an SGPR
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

  if (kt0 < kt1)
    stage_tiles<Cfg::TILE_BYTES>(kbase + (size_t)kt0 * Cfg::TILE_BYTES,
                                 vbase + (size_t)kt0 * Cfg::TILE_BYTES, stage0,
                                 stage0 + Cfg::TILE_BYTES, w, lane);

  // One key tile; ST is the stage holding it (compile-time, so every LDS access
  // names its own object).
  auto tile = [&](auto stc, int kt) {
    constexpr int ST = decltype(stc)::value;
    unsigned char* cur = ST == 0 ? stage0 : stage1;
    unsigned char* nxt = ST == 0 ? stage1 : stage0;
    wait_vmem();
    __syncthreads();  // tile kt is in LDS; every wave is done with the other stage
    if (STAGES == 2 && kt + 1 < kt1)
      stage_tiles<Cfg::TILE_BYTES>(kbase + (size_t)(kt + 1) * Cfg::TILE_BYTES,
                                   vbase + (size_t)(kt + 1) * Cfg::TILE_BYTES, nxt,
                                   nxt + Cfg::TILE_BYTES, w, lane);
    const uint4* k_lds = reinterpret_cast<const uint4*>(cur);
    uint4* v_lds = reinterpret_cast<uint4*>(cur + Cfg::TILE_BYTES);
    if ((kt + 1) * kNTile > kend) {
      // positions at or beyond start + R may hold anything: zero their values
      for (int i = tid; i < Cfg::VVEC; i += 256) {
        const int gi = i / D;  // vector i of the tile: group gi holds E positions
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
        if ((keep[0] & keep[1] & keep[2] & keep[3]) != ~0u) {
          uint4 v = v_lds[i];
          v.x &= keep[0]; v.y &= keep[1]; v.z &= keep[2]; v.w &= keep[3];
          v_lds[i] = v;
        }
      }
      __syncthreads();
    }

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
    float tile_max[2];
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
      tile_max[mb] = mx;
    }
    // Lazy rescale: the reference max of a column moves only when the tile
    // max exceeds it by more than kRescaleSlack (log2 units), so weights stay
    // below 2^kRescaleSlack and the accumulator pass below runs only in the
    // rare tiles where some column of the wave needs it.  acc and l always
    // share one reference, so the result is the same softmax.
    bool need = false;
    float alpha[2] = {1.f, 1.f};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      if (tile_max[mb] > m_run[mb] + kRescaleSlack) {
        alpha[mb] = fast_exp2(m_run[mb] - tile_max[mb]);   // 0 when m_run is -inf
        m_run[mb] = tile_max[mb];
        l_run[mb] *= alpha[mb];
        need = true;
      }
    }
    if (__any(need)) {
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] *= alpha[mb];
    }
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const float m_use = m_run[mb] == -INFINITY ? 0.f : m_run[mb];
      float ls = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(sacc[kb][mb][i] - m_use);
          sacc[kb][mb][i] = pv;
          ls += pv;
        }
      l_run[mb] += ls;
    }

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
    if (STAGES == 1 && kt + 1 < kt1) {
      __syncthreads();  // every wave is done with the only stage
      stage_tiles<Cfg::TILE_BYTES>(kbase + (size_t)(kt + 1) * Cfg::TILE_BYTES,
                                   vbase + (size_t)(kt + 1) * Cfg::TILE_BYTES, cur,
                                   cur + Cfg::TILE_BYTES, w, lane);
    }
  };
  for (int kt = kt0; kt < kt1; kt += 2) {
    tile(std::integral_constant<int, 0>(), kt);
    if (kt + 1 < kt1) tile(std::integral_constant<int, STAGES == 2 ? 1 : 0>(), kt + 1);
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
      // acc [tile][S][128 columns][D]; (m, l) [tile][128 columns][S][2]
      const size_t tile_id = ((size_t)b * Hkv + g) * m_tiles + mt;
      const int col = m_col[mb] - m_base;
      float* pp = part + ((tile_id * S + split) * kMTile + col) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc_o[db][mb];
        *reinterpret_cast<float4*>(pp + 16 * db + 4 * lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (lg == 0) {
        float* ml = part_ml + ((tile_id * kMTile + col) * S + split) * 2;
        ml[0] = m_run[mb];
        ml[1] = lt;
      }
    }
  }
}

// Combines the S split partials of 16 columns of one M-tile.  Thread (c, v)
// owns column c and the float4 dims 4 v + 64 j; splits are summed in order.
template <int D>
__global__ __launch_bounds__(256) void prefill_merge_kernel(
    const float* __restrict__ part, const float* __restrict__ part_ml, float* __restrict__ out,
    int Hq, int Hkv, int R, int m_tiles, int S) {
  __shared__ float wgt[16][kMaxSplits];
  __shared__ float inv_l[16];
  const int mt = blockIdx.x >> 3, cg = blockIdx.x & 7;
  const int g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv;
  const int M_total = R * G;
  const int tid = threadIdx.x;
  const size_t tile_id = ((size_t)b * Hkv + g) * m_tiles + mt;
  if (tid < 16) {
    const float* ml = part_ml + (tile_id * kMTile + cg * 16 + tid) * S * 2;
    float M = -INFINITY;
    for (int s = 0; s < S; ++s) M = fmaxf(M, ml[2 * s]);
    float L = 0.f;
    for (int s = 0; s < S; ++s) {
      const float f = ml[2 * s] == -INFINITY ? 0.f : fast_exp2(ml[2 * s] - M);
      wgt[tid][s] = f;
      L += f * ml[2 * s + 1];
    }
    inv_l[tid] = 1.f / L;
  }
  __syncthreads();
  const int c = tid >> 4, v = tid & 15;
  const int col = cg * 16 + c;
  const int m = mt * kMTile + col;
  if (m >= M_total) return;
  const int row = m / G, hh = m % G;
  float* op = out + (((size_t)b * R + row) * Hq + g * G + hh) * D;
  const float* pc = part + (tile_id * S * kMTile + col) * D;
  const size_t PS = (size_t)kMTile * D;  // stride between splits
  const float il = inv_l[c];
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    const int d = 4 * v + 64 * j;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    int s = 0;
    for (; s + 8 <= S; s += 8) {
      float4 t[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) t[k] = *reinterpret_cast<const float4*>(pc + (s + k) * PS + d);
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float f = wgt[c][s + k];
        a.x += f * t[k].x; a.y += f * t[k].y; a.z += f * t[k].z; a.w += f * t[k].w;
      }
    }
    for (; s < S; ++s) {
      const float f = wgt[c][s];
      const float4 t = *reinterpret_cast<const float4*>(pc + s * PS + d);
      a.x += f * t.x; a.y += f * t.y; a.z += f * t.z; a.w += f * t.w;
    }
    *reinterpret_cast<float4*>(op + d) = make_float4(a.x * il, a.y * il, a.z * il, a.w * il);
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
  auto kern = prefill_kernel<D, BF16>;
  dim3 grid(p.m_tiles * p.splits, s.num_kv_heads, s.batch);
  float* part = reinterpret_cast<float*>(ws);
  float* part_ml = part + (size_t)s.batch * s.num_kv_heads * p.m_tiles * p.splits * kMTile * D;
  hipLaunchKernelGGL(kern, grid, dim3(256), 0, st, q, kc, vc, out, part, part_ml,
                     s.num_q_heads, s.num_kv_heads, s.capacity, start, R, p.m_tiles, p.splits,
                     scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.splits > 1) {
    hipLaunchKernelGGL(prefill_merge_kernel<D>, dim3(p.m_tiles * 8, s.num_kv_heads, s.batch),
                       dim3(256), 0, st, part, part_ml, out, s.num_q_heads, s.num_kv_heads, R,
                       p.m_tiles, p.splits);
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
            (size_t)(s.head_dim + 2) * sizeof(float);
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
                         (size_t)(s.head_dim + 2) * sizeof(float);
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
