// Chunked prefill on MFMA: rows start .. start+R-1 attend causally to the
// cache of their session.
//
// Tiling.  One workgroup owns an M-tile of 128 (row, query head) pairs of one
// KV head -- for 8 heads per KV head that is 16 consecutive rows x 8 heads --
// and a range of 64-position key tiles (one split of the causal key range).
// Each K / V tile is staged once in LDS and read by all the workgroup's
// waves, so every K / V row is fetched once per M-tile, i.e. once per 128 / G
// chunk rows and shared by every query head of the group.  bf16 caches: 8
// waves on v_mfma_f32_32x32x16_bf16 (Q and P rounded to bf16, f32
// accumulation); f32 caches: 4 waves on v_mfma_f32_16x16x4_f32, each owning
// 32 of the 128 M columns.
//
// Products.  Scores are computed transposed, S^T = K . Q^T (M = keys,
// N = (row, head) pairs), and values as O^T = V^T . P^T (M = dims).  In the
// MFMA accumulator layout a lane then holds one (row, head) column and a set
// of keys / dims, so the running max, the running sum and any rescale of the
// accumulator are lane-local, and the exponentiated S^T registers are already
// the B operand of the value product: the V layouts group positions exactly
// as a lane holds them.
//
// Softmax.  Online (flash-style) in f32, log2 domain.  Only tiles that cross
// a row's causal limit are masked; tiles above every row's limit are not
// visited.  Positions at or beyond start + R are zeroed in LDS so that
// whatever the cache holds there cannot reach a result.
//
// Splits.  When the key range is split, each split writes a partial (m, l,
// acc) and a second kernel combines them in fixed split order.
#include <cfloat>
#include <type_traits>
#include <vector>

#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

namespace {

constexpr int kMTile = 128;
constexpr int kNTile = 64;
constexpr int kMaxSplits = 64;
constexpr float kRescaleSlack = 8.f;  // log2 units: weights stay below 256
constexpr float kFrameSlack = 32.f;   // log2 units (8-wave kernel, see prefill_mtile_kernel)

typedef __attribute__((ext_vector_type(4))) float v4f;

// Tiles of f32 (BF16 false) or bf16 values: 16-byte vectors of E elements.
template <int D, bool BF16>
struct PrefillCfg {
  static constexpr int E = Elem<BF16>::E;
  static constexpr int KVEC = D / E * kNTile;            // 16-byte vectors per K tile
  static constexpr int VVEC = kNTile / E * D;            // 16-byte vectors per V tile
  static constexpr int TILE_BYTES = KVEC * 16;           // same for V
  static constexpr int NDB = D / 16;                     // 16-dim output blocks
  // f32 kernels: K and V tiles double-buffered separately (4 tiles, the
  // pipelined kernel) when that fits the 160 KiB of LDS; otherwise one K+V
  // stage (the sequential kernel).
  static constexpr bool PIPE = 4 * TILE_BYTES <= 160 * 1024;
};

// A cache slab as a buffer resource (see buffer_rsrc).
struct TileSrc {
  __amdgpu_buffer_rsrc_t rsrc;
};

__device__ __forceinline__ TileSrc tile_src(const void* slab, size_t bytes) {
  TileSrc src;
  src.rsrc = buffer_rsrc(slab, bytes);
  return src;
}

// Asynchronous copy of tile `tile` (TILE_BYTES contiguous bytes of the slab)
// into LDS: every wave instruction moves 1 KiB, lane l's 16 bytes landing at
// the wave's LDS base + 16 l.
template <int TILE_BYTES, int NT = 256>
__device__ __forceinline__ void load_tile(const TileSrc& src, int tile, unsigned char* dst, int w,
                                          int lane) {
  constexpr int PER_THREAD = TILE_BYTES / (NT * 16);
#pragma unroll
  for (int i = 0; i < PER_THREAD; ++i) {
    const int off = (i * NT + w * 64) * 16;
    dma16(src.rsrc, dst + off, tile * TILE_BYTES + off + lane * 16);
  }
}

// The sessions of one prefill launch.  Session i: rows start[i] ..
// start[i] + rows[i] - 1, stored at packed rows row0[i] .. of q and out; cache
// slab b[i]; m_tiles[i] M-tiles and splits[i] key-range splits per KV head;
// partial slots from slot0[i] (KV head, m-tile, split order); work items
// item0[i] .. item0[i + 1] - 1.  A uniform chunk over B sessions is B equal
// entries (launched kChunkSessions at a time).
constexpr int kChunkSessions = 32;
struct ChunkArg {
  int n;
  int b[kChunkSessions], start[kChunkSessions], rows[kChunkSessions], m_tiles[kChunkSessions];
  int splits[kChunkSessions], row0[kChunkSessions], slot0[kChunkSessions];
  int item0[kChunkSessions + 1];
};

// Per-block constants of the tiling.  The block's session: rows start ..
// start + R - 1 at packed rows row0 .. of q / out, m_tiles M-tiles and S
// splits per KV head; slot is its partial slot of split 0 (one slot holds
// one split's 128-column partial).
struct Tiling {
  int mt, split, g, b, G, M_total, lr, lg, w, lane, tid;
  int m_base, row_lo, kt0, kt1, kend;
  int start, R, m_tiles, S, row0;
  long long slot;
  int m_col[2], row_col[2];
  bool valid_col[2];
};

// Block -> (session, KV head, m-tile, split).  The sessions' work items are
// numbered session by session, each (KV head, m-tile)-major with the split
// fastest, and dealt to the 8 XCDs in contiguous runs: consecutive
// workgroups go to the XCDs round-robin, so block x runs on XCD x % 8 and
// takes item (x % 8) * per + x / 8.  The splits of an m-tile then share one
// XCD, whose L2 serves their common Q rows (read once per workgroup) while
// the key tiles stream past.  The grid is padded to 8 * per blocks; blocks
// past the last item return false.
__device__ __forceinline__ bool make_tiling(const ChunkArg& ca, int Hq, int Hkv, Tiling& t) {
  const int items = ca.item0[ca.n];
  const int per = (items + 7) >> 3;
  const int x = blockIdx.x;
  const int item = (x & 7) * per + (x >> 3);
  if (item >= items) return false;
  int i = 0;
  while (item >= ca.item0[i + 1]) ++i;
  const int S = ca.splits[i], m_tiles = ca.m_tiles[i];
  const int local = item - ca.item0[i];
  const int gm = local / S;  // (KV head, m-tile)
  t.split = local - gm * S;
  t.g = gm / m_tiles;
  t.mt = gm - t.g * m_tiles;
  t.b = ca.b[i];
  t.start = ca.start[i];
  t.R = ca.rows[i];
  t.m_tiles = m_tiles;
  t.S = S;
  t.row0 = ca.row0[i];
  t.slot = (long long)ca.slot0[i] + (long long)gm * S;
  const int start = t.start, R = t.R;
  t.G = Hq / Hkv;
  t.M_total = R * t.G;
  t.tid = threadIdx.x;
  t.lane = t.tid & 63;
  t.w = __builtin_amdgcn_readfirstlane(t.tid >> 6);  // wave index, kept in an SGPR
  t.lr = t.lane & 15;
  t.lg = t.lane >> 4;
  t.m_base = t.mt * kMTile;
  t.row_lo = t.m_base / t.G;
  const int row_hi = min(R - 1, (t.m_base + kMTile - 1) / t.G);
  const int nkt = (start + row_hi) / kNTile + 1;
  // split * nkt stays below 2^31 (at most 64 splits of 2048 key tiles)
  t.kt0 = t.split * nkt / S;
  t.kt1 = (t.split + 1) * nkt / S;
  t.kend = start + R;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    t.m_col[mb] = t.m_base + t.w * 32 + mb * 16 + t.lr;
    t.valid_col[mb] = t.m_col[mb] < t.M_total;
    t.row_col[mb] = t.valid_col[mb] ? t.m_col[mb] / t.G : 0;
  }
  return true;
}

// The 4-wave kernels below (f32 caches, v_mfma_f32_16x16x4f32): wave w owns
// columns 32 w .. 32 w + 31 of the M-tile as two 16-column blocks mb; lane
// (lr, lg) = (l % 16, l / 16).

// Stationary Q^T operand: this lane's slice of its two columns.
template <int D>
__device__ __forceinline__ void load_q(const Tiling& t, const float* __restrict__ q, int R, int Hq,
                                       v4f (&qreg)[2][D / 16]) {
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int m = t.m_col[mb];
    const float* qp = q + (((size_t)t.row0 + m / t.G) * Hq + t.g * t.G + m % t.G) * D;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      v4f a = {0.f, 0.f, 0.f, 0.f};
      if (t.valid_col[mb]) {
        const float4 v = *reinterpret_cast<const float4*>(qp + 16 * ks + 4 * t.lg);
        a[0] = v.x; a[1] = v.y; a[2] = v.z; a[3] = v.w;
      }
      qreg[mb][ks] = a;
    }
  }
}

// S^T = K . Q^T for one 64-position tile: 4 key blocks x 2 column blocks.
template <int D>
__device__ __forceinline__ void qk_tile(const uint4* __restrict__ k_lds, const v4f (&qreg)[2][D / 16],
                                        v4f (&sacc)[4][2], int lr, int lg) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) sacc[kb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
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
        for (int u = 0; u < 4; ++u)
          sacc[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], qreg[mb][c4][u], sacc[kb][mb], 0, 0, 0);
    }
  }
}

// Causal mask (only on tiles that cross a row's limit) and online softmax of
// one tile: turns the scores into weights in place, updates m and l, and
// returns the accumulator rescale factors (1 where the reference max stayed).
__device__ __forceinline__ void softmax_tile(const Tiling& t, int kt, int start, float sl2e,
                                             v4f (&sacc)[4][2], float (&m_run)[2],
                                             float (&l_run)[2], float (&alpha)[2]) {
  const bool diag = kt * kNTile + kNTile - 1 > start + t.row_lo;
  float tile_max[2];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    const int lim = start + t.row_col[mb];
    // scores to the log2 domain first, so a column's largest term is
    // exactly exp2(0) = 1
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float sv = sacc[kb][mb][i] * sl2e;
        if (diag) {
          const int key = kt * kNTile + 16 * kb + 4 * t.lg + i;
          if (key > lim || !t.valid_col[mb]) sv = -INFINITY;
        }
        sacc[kb][mb][i] = sv;
        mx = fmaxf(mx, sv);
      }
    mx = fmaxf(mx, xor_shfl(mx, 16));
    mx = fmaxf(mx, xor_shfl(mx, 32));
    tile_max[mb] = mx;
  }
  // Lazy rescale: a column's reference max moves only when the tile max
  // exceeds it by more than kRescaleSlack (log2 units), so weights stay below
  // 2^kRescaleSlack and the accumulator pass (rescale_acc) runs only in the
  // rare tiles where some column of the wave needs it.  acc and l always
  // share one reference, so the result is the same softmax.
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    alpha[mb] = 1.f;
    if (tile_max[mb] > m_run[mb] + kRescaleSlack) {
      alpha[mb] = fast_exp2(m_run[mb] - tile_max[mb]);  // 0 when m_run is -inf
      m_run[mb] = tile_max[mb];
      l_run[mb] *= alpha[mb];
    }
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
}

// Applies the rescale factors softmax_tile chose (a uniform branch: skipped
// when no column of the wave moved its reference max).
template <int NDB>
__device__ __forceinline__ void rescale_acc(const float (&alpha)[2], v4f (&acc_o)[NDB][2]) {
  if (__any(alpha[0] != 1.f || alpha[1] != 1.f)) {
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] *= alpha[mb];
  }
}

// O^T += V^T . P^T for one tile (P = the weights left in sacc).
template <int D>
__device__ __forceinline__ void pv_tile(const uint4* __restrict__ v_lds, const v4f (&p)[4][2],
                                        v4f (&acc_o)[D / 16][2], int lr, int lg) {
#pragma unroll
  for (int db = 0; db < D / 16; ++db)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 a = v_lds[(4 * kb + lg) * D + 16 * db + lr];
      const float av[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                           __uint_as_float(a.w)};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          acc_o[db][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], p[kb][mb][u], acc_o[db][mb], 0, 0, 0);
    }
}

// Positions at or beyond kend may hold anything: zero their values in the
// staged V tile kt (every thread of the block takes part).
template <int D, bool BF16, int NT = 256>
__device__ __forceinline__ void zero_v_beyond(uint4* v_lds, int kt, int kend, int tid) {
  constexpr int VVEC = PrefillCfg<D, BF16>::VVEC;
  for (int i = tid; i < VVEC; i += NT) {
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
}

// Causality under non-finite values.  The columns of a tile that crosses a
// row's causal limit share one value product, in which a key past a
// column's limit carries weight 0 -- and 0 * NaN or 0 * inf is NaN.  So a
// non-finite V value at a position that some column of the tile cannot see
// must not enter the shared product: such tiles are scanned, those values
// are zeroed for the product, and each reaches only the columns whose limit
// reaches it, as the IEEE sum would: acc + w * v is NaN for a NaN v, for
// +inf and -inf together and for w = 0; otherwise it is +-inf.  Positions at
// or below lo are seen by every column of the tile; positions at or beyond
// hi (the chunk's end) are zeroed already.  (Class codes and tables: see
// class_bf16.)
//
// Any non-finite element in a 16-byte vector of the V layout.
template <bool BF16>
__device__ __forceinline__ bool any_nonfinite(const uint4& v) {
  if constexpr (BF16) {
    auto two = [](uint32_t w) { return bf16_nonfinite(w) || bf16_nonfinite(w >> 16); };
    return two(v.x) || two(v.y) || two(v.z) || two(v.w);
  } else {
    return f32_nonfinite(v.x) || f32_nonfinite(v.y) || f32_nonfinite(v.z) || f32_nonfinite(v.w);
  }
}

// Scan of the staged V tile kt, this thread's share of its 16-byte vectors:
// the mask of tile positions (bit p - 64 kt) holding a non-finite value with
// lo < p < hi.  With MARK it also zeroes those values in LDS and ORs their
// classes into the table.
template <int D, bool BF16, int NT, bool MARK>
__device__ __forceinline__ uint64_t nonfinite_v(uint4* v_lds, int kt, int lo, int hi, int tid,
                                                uint32_t* tab) {
  constexpr int VVEC = PrefillCfg<D, BF16>::VVEC;
  constexpr int NE = BF16 ? 8 : 4;
  uint64_t bits = 0;
#pragma unroll 1
  for (int i = tid; i < VVEC; i += NT) {
    const uint4 v = v_lds[i];
    if (!any_nonfinite<BF16>(v)) continue;
    const int gi = i / D, d = i - gi * D;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      int pl;
      uint32_t x;
      if constexpr (BF16) {
        pl = vbf16_pos(gi >> 2, gi & 3, e);
        x = (w[e >> 1] >> (16 * (e & 1))) & 0xffffu;
      } else {
        pl = gi * 4 + e;
        x = w[e];
      }
      const int p = kt * kNTile + pl;
      const bool nf = BF16 ? bf16_nonfinite(x) : f32_nonfinite(x);
      if (nf && p > lo && p < hi) {
        bits |= 1ull << pl;
        if constexpr (MARK) {
          atomicOr(tab + pl * (D / 16) + d / 16,
                   (BF16 ? class_bf16(x) : class_f32(x)) << (2 * (d % 16)));
          if constexpr (BF16) w[e >> 1] &= ~(0xffffu << (16 * (e & 1)));
          else w[e] = 0u;
        }
      }
    }
    if (MARK) v_lds[i] = make_uint4(w[0], w[1], w[2], w[3]);
  }
  return bits;
}

// The block's mask of such positions in tile kt (an OR over the waves
// through nfm[2 * waves]); when it is not 0 (rare), the flagged values are
// zeroed in LDS and their classes entered in tab (rows of flagged positions
// cleared first).  Every thread calls this; after it returns the tile and
// the table are visible to every wave.
template <int D, bool BF16, int NT>
__device__ __forceinline__ uint64_t sanitize_tile(uint4* v_lds, int kt, int lo, int hi, int tid,
                                                  uint32_t* nfm, uint32_t* tab) {
  constexpr int NW = NT / kWave;
  const uint64_t bits = nonfinite_v<D, BF16, NT, false>(v_lds, kt, lo, hi, tid, tab);
  const uint32_t b0 = wave_or((uint32_t)bits), b1 = wave_or((uint32_t)(bits >> 32));
  const int w = tid / kWave;
  if ((tid & (kWave - 1)) == 0) {
    nfm[2 * w] = b0;
    nfm[2 * w + 1] = b1;
  }
  __syncthreads();
  uint64_t nf = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) nf |= (uint64_t)nfm[2 * k] | ((uint64_t)nfm[2 * k + 1] << 32);
  if (nf != 0) {
    for (int i = tid; i < kNTile * (D / 16); i += NT)
      if ((nf >> (i / (D / 16))) & 1) tab[i] = 0u;
    __syncthreads();
    nonfinite_v<D, BF16, NT, true>(v_lds, kt, lo, hi, tid, tab);
    __syncthreads();
  }
  return nf;
}

// f32 kernels: the flagged values of tile kt, into the columns that see them.
// p: the tile's weights (lane (lr, lg) holds keys 16 kb + 4 lg + i of its
// columns), acc_o: dims 16 db + 4 lg + 0..3.
template <int D>
__device__ __forceinline__ void add_nonfinite_f32(uint64_t nf, int kt, const Tiling& t, int start,
                                                  const v4f (&p)[4][2], const uint32_t* tab,
                                                  v4f (&acc_o)[D / 16][2]) {
  // [mb][db / 4]: dims 16 db + 4 lg + 0..3 at bits 8 (db % 4) .., 2 bits each
  uint32_t cls[2][D / 64];
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int j = 0; j < D / 64; ++j) cls[mb][j] = 0u;
  while (nf != 0) {
    const int pl = __builtin_ctzll(nf);
    nf &= nf - 1;
    const int key = kt * kNTile + pl;
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      float sel = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) sel = (kb == (pl >> 4) && i == (pl & 3)) ? p[kb][mb][i] : sel;
      const float wgt = __shfl(sel, t.lr + 16 * ((pl >> 2) & 3), kWave);
      if (!t.valid_col[mb] || key > start + t.row_col[mb]) continue;
#pragma unroll
      for (int db = 0; db < D / 16; ++db) {
        uint32_t byte = (tab[pl * (D / 16) + db] >> (8 * t.lg)) & 0xffu;
        if (wgt == 0.f) byte = all_nan(byte);
        cls[mb][db >> 2] |= byte << (8 * (db & 3));
      }
    }
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb)
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      apply_classes<4>(cls[mb][db >> 2] >> (8 * (db & 3)), acc_o[db][mb], 0);
}

// Epilogue: normalised output (one split) or the split's partial.
template <int D>
__device__ __forceinline__ void store_result(const Tiling& t, float* __restrict__ out,
                                             float* __restrict__ part, float* __restrict__ part_ml,
                                             const v4f (&acc_o)[D / 16][2], const float (&m_run)[2],
                                             const float (&l_run)[2], int R, int Hq, int Hkv,
                                             int m_tiles, int S) {
  constexpr int NDB = D / 16;
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) {
    float lt = l_run[mb];
    lt += xor_shfl(lt, 16);
    lt += xor_shfl(lt, 32);
    if (!t.valid_col[mb]) continue;
    if (S == 1) {
      const int m = t.m_col[mb];
      float* op = out + (((size_t)t.row0 + m / t.G) * Hq + t.g * t.G + m % t.G) * D;
      const float inv = 1.f / lt;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc_o[db][mb] * inv;
        *reinterpret_cast<float4*>(op + 16 * db + 4 * t.lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
    } else {
      // acc [slot][128 columns][D]; (m, l) [tile][128 columns][S][2]
      const int col = t.m_col[mb] - t.m_base;
      float* pp = part + (((size_t)t.slot + t.split) * kMTile + col) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const v4f o = acc_o[db][mb];
        *reinterpret_cast<float4*>(pp + 16 * db + 4 * t.lg) = make_float4(o[0], o[1], o[2], o[3]);
      }
      if (t.lg == 0) {
        float* ml = part_ml + ((size_t)t.slot * kMTile + (size_t)col * S + t.split) * 2;
        ml[0] = m_run[mb];
        ml[1] = lt;
      }
    }
  }
}

// Scores of the next tile fused with the softmax of the current one.  The
// K-operand reads run one chunk ahead in registers; each chunk (one k-step of
// the score product: 8 MFMAs with bf16) carries a slice of the softmax work,
// and a scheduling fence closes it, so the VALU work of the softmax issues in
// the cycles between MFMA issues instead of after all of them.
//   softmax phases: 0, 1 scale + mask + local max of column block 0 / 1;
//   2 cross-lane max; 3 reference-max update; 4..7 exponentials of key
//   block 0..3.
template <int D>
__device__ __forceinline__ void qk_next_softmax_cur(
    const Tiling& t, const uint4* __restrict__ k_lds, const v4f (&qreg)[2][D / 16],
    v4f (&nxt)[4][2], v4f (&cur)[4][2], int kt, int start, float sl2e, float (&m_run)[2],
    float (&l_run)[2], float (&alpha)[2]) {
  constexpr int NKS = D / 16;  // k-steps of the score product
  const int lr = t.lr, lg = t.lg;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) nxt[kb][mb] = v4f{0.f, 0.f, 0.f, 0.f};
  const bool diag = kt * kNTile + kNTile - 1 > start + t.row_lo;
  float lmax[2] = {-INFINITY, -INFINITY};
  float ls[2] = {0.f, 0.f};
  float m_use[2];
  uint4 kbuf[2][4];
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) kbuf[0][kb] = k_lds[(4 * 0 + lg) * 64 + 16 * kb + lr];

  auto phase = [&](int ph) {
    if (ph == 0 || ph == 1) {
      const int mb = ph;
      const int lim = start + t.row_col[mb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // scores to the log2 domain first, so a column's largest term is
          // exactly exp2(0) = 1
          float sv = cur[kb][mb][i] * sl2e;
          if (diag) {
            const int key = kt * kNTile + 16 * kb + 4 * lg + i;
            if (key > lim || !t.valid_col[mb]) sv = -INFINITY;
          }
          cur[kb][mb][i] = sv;
          lmax[mb] = fmaxf(lmax[mb], sv);
        }
    } else if (ph == 2) {
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        lmax[mb] = fmaxf(lmax[mb], xor_shfl(lmax[mb], 16));
        lmax[mb] = fmaxf(lmax[mb], xor_shfl(lmax[mb], 32));
      }
    } else if (ph == 3) {
      // Lazy rescale: a column's reference max moves only when the tile max
      // exceeds it by more than kRescaleSlack (log2 units); weights stay
      // below 2^kRescaleSlack.  acc and l share one reference throughout.
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        alpha[mb] = 1.f;
        if (lmax[mb] > m_run[mb] + kRescaleSlack) {
          alpha[mb] = fast_exp2(m_run[mb] - lmax[mb]);  // 0 when m_run is -inf
          m_run[mb] = lmax[mb];
          l_run[mb] *= alpha[mb];
        }
        m_use[mb] = m_run[mb] == -INFINITY ? 0.f : m_run[mb];
      }
    } else {
      const int kb = ph - 4;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float pv = fast_exp2(cur[kb][mb][i] - m_use[mb]);
          cur[kb][mb][i] = pv;
          ls[mb] += pv;
        }
    }
  };

#pragma unroll
  for (int ks = 0; ks < NKS; ++ks) {
    if (ks + 1 < NKS) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        kbuf[(ks + 1) & 1][kb] = k_lds[(4 * (ks + 1) + lg) * 64 + 16 * kb + lr];
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const uint4 a = kbuf[ks & 1][kb];
      const float av[4] = {__uint_as_float(a.x), __uint_as_float(a.y), __uint_as_float(a.z),
                           __uint_as_float(a.w)};
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int u = 0; u < 4; ++u)
          nxt[kb][mb] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[u], qreg[mb][ks][u], nxt[kb][mb], 0, 0, 0);
    }
    // softmax phases assigned to this chunk (all 8 spread over NKS chunks)
#pragma unroll
    for (int ph = 0; ph < 8; ++ph)
      if (ph * NKS / 8 == ks) phase(ph);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int mb = 0; mb < 2; ++mb) l_run[mb] += ls[mb];
}

// Pipelined prefill.  K runs one tile ahead of V: while the weights of tile i
// are formed (VALU), the score MFMAs of tile i+1 are already issued, and the
// copies of K(i+2) and V(i+1) are in flight.  K and V each have two LDS
// buffers; the loop is unrolled by two so every access names its buffer.
template <int D>
__global__ __launch_bounds__(256) void prefill_pipe_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    float* __restrict__ part_ml, int Hq, int Hkv, int C, const ChunkArg ca, float sl2e) {
  using Cfg = PrefillCfg<D, false>;
  constexpr int NDB = Cfg::NDB, TB = Cfg::TILE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char kb0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char kb1[TB];
  __shared__ __attribute__((aligned(16))) unsigned char vb0[TB];
  __shared__ __attribute__((aligned(16))) unsigned char vb1[TB];
  __shared__ uint32_t nfm[8];                  // non-finite value masks, [wave][2]
  __shared__ uint32_t nf_tab[kNTile * D / 16];  // and their classes

  Tiling t;
  if (!make_tiling(ca, Hq, Hkv, t)) return;
  const int start = t.start, R = t.R, m_tiles = t.m_tiles, S = t.S;
  const size_t slab = ((size_t)t.b * Hkv + t.g) * (size_t)C * D;  // elements
  const TileSrc ksrc = tile_src(reinterpret_cast<const unsigned char*>(k_cache) + slab * 4, (size_t)C * D * 4);
  const TileSrc vsrc = tile_src(reinterpret_cast<const unsigned char*>(v_cache) + slab * 4, (size_t)C * D * 4);
  const int n = t.kt1 - t.kt0;

  v4f qreg[2][D / 16];
  v4f acc_o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  v4f sa[4][2], sb[4][2];

  if (n > 0) {
    load_tile<TB>(ksrc, t.kt0, kb0, t.w, t.lane);
    load_q<D>(t, q, R, Hq, qreg);
    wait_vmem();
    __syncthreads();
    load_tile<TB>(vsrc, t.kt0, vb0, t.w, t.lane);
    if (n > 1) load_tile<TB>(ksrc, t.kt0 + 1, kb1, t.w, t.lane);
    qk_tile<D>(reinterpret_cast<const uint4*>(kb0), qreg, sa, t.lr, t.lg);
  }

  // step i: V(i) in vb[i&1], K(i+1) in kb[(i+1)&1], scores of tile i in cur
  auto step = [&](auto par, int i, v4f (&cur)[4][2], v4f (&nxt)[4][2]) {
    constexpr int P = decltype(par)::value;
    unsigned char* k_next = P == 0 ? kb1 : kb0;   // holds K(i+1)
    unsigned char* k_free = P == 0 ? kb0 : kb1;   // held K(i): free for K(i+2)
    unsigned char* v_cur = P == 0 ? vb0 : vb1;    // holds V(i)
    unsigned char* v_free = P == 0 ? vb1 : vb0;   // held V(i-1): free for V(i+1)
    const int kt = t.kt0 + i;
    wait_vmem();
    __syncthreads();  // V(i), K(i+1) landed; every wave is done with step i-1
    if (i + 2 < n) load_tile<TB>(ksrc, kt + 2, k_free, t.w, t.lane);
    if (i + 1 < n) load_tile<TB>(vsrc, kt + 1, v_free, t.w, t.lane);
    if ((kt + 1) * kNTile > t.kend) {
      zero_v_beyond<D, false>(reinterpret_cast<uint4*>(v_cur), kt, t.kend, t.tid);
      __syncthreads();
    }
    // a tile crossing a row's limit: non-finite values only where seen
    const bool cross = kt * kNTile + kNTile - 1 > start + t.row_lo;
    uint64_t nf = 0;
    if (cross)
      nf = sanitize_tile<D, false, 256>(reinterpret_cast<uint4*>(v_cur), kt, start + t.row_lo,
                                        t.kend, t.tid, nfm, nf_tab);
    // The next tile's score MFMAs and this tile's softmax are independent
    // and run interleaved (the last step computes one spare tile of scores
    // from a stale buffer, which is never used).
    float alpha[2];
    qk_next_softmax_cur<D>(t, reinterpret_cast<const uint4*>(k_next), qreg, nxt, cur, kt,
                                 start, sl2e, m_run, l_run, alpha);
    rescale_acc<NDB>(alpha, acc_o);
    pv_tile<D>(reinterpret_cast<const uint4*>(v_cur), cur, acc_o, t.lr, t.lg);
    if (nf != 0) add_nonfinite_f32<D>(nf, kt, t, start, cur, nf_tab, acc_o);
  };
  for (int i = 0; i < n; i += 2) {
    step(std::integral_constant<int, 0>(), i, sa, sb);
    if (i + 1 < n) step(std::integral_constant<int, 1>(), i + 1, sb, sa);
  }
  store_result<D>(t, out, part, part_ml, acc_o, m_run, l_run, R, Hq, Hkv, m_tiles, S);
}

// ============================================================================
// bf16 and int8-K caches: 32x32 MFMAs, 8 waves (prefill_mtile_kernel).
//
// Work split.  Wave w takes column block cb = w & 3 (M columns 32 cb ..
// 32 cb + 31 of the tile) and half kh = w >> 2: it scores keys 32 kh ..
// 32 kh + 31 of every 64-position tile and owns output dims kh D/2 ..
// kh D/2 + D/2 - 1.  Waves w and w ^ 4 (the pair of a column block) exchange
// their bf16 weights through LDS (2 KiB per wave and tile) and share one
// softmax frame.  Two waves per SIMD, at most 256 registers each, so one
// wave's LDS and dependency waits are covered by the other's work.  Lane l
// holds column l % 32 of the block (half h = l / 32).
//   S^T = K . Q^T per 16-dim step ks: A = K[32 kh + l % 32][16 ks + 8 h .. + 7]
//     (16 bytes of the K layout), B = Q^T, stationary in registers and
//     pre-multiplied by scale * log2(e), so scores arrive in the log2 domain.
//     Accumulator register 4 a + e holds key 32 kh + 8 a + 4 h + e.
//   O^T += V^T . P^T per 16-key step (kb, s): A = V group 4 kb + 2 s + h at dim
//     32 db + l % 32 (16 bytes of the V layout), B = the weights of keys
//     {32 kb + 16 s + 4 h + 0..3, 32 kb + 16 s + 8 + 4 h + 0..3} of the lane's
//     column: accumulator registers 8 s .. 8 s + 7 of the scores of key half
//     kb, rounded to bf16 -- this wave's own for kb = kh, the partner's (same
//     lane, from LDS) for kb = 1 - kh.
// Pipeline.  Step i issues, on the matrix pipe, the scores of tile i+1 and the
// value product of tile i-1 (16 + 16 MFMAs per wave for D = 256) and, on the
// vector pipe between them, the softmax of tile i.  K(i+2) and V(i) stream
// into LDS meanwhile; K, V and the weight exchange each have two buffers.
//
// int8-K caches (I8).  K tiles hold int8 codes (64 D bytes, the K layout with
// 16 codes per vector) followed in LDS by the tile's 64 row scales (256
// bytes, staged by 16 lanes of wave 0).  Q is quantised per column as K is
// (amax over the column's D values: this lane's half and lane l ^ 32's), its
// codes stationary in registers.  Scores use v_mfma_i32_32x32x32_i8 per
// 32-dim step: A = the 16 codes of key 32 kh + l % 32 at dims 32 ks + 16 h ..
// (one 16-byte vector of the K layout, at the same LDS index as a bf16 step's
// operand), B = the column's 16 codes at those dims; the accumulator layout is
// the bf16 one.  Half as many score MFMAs (on even chunks of a step), and
// half the K bytes in LDS reads and DMA.  After a tile's last score MFMA the
// integer dots become (float) dot * (s_q * scale * log2 e) * s_key, so the
// softmax and the value product are the bf16 path's.
//
// Reference frame.  A column's weights are exp2(s - m_ref), where m_ref is the
// largest score of the first tile of the range (both halves; a column that
// sees any key of the range sees that tile's first key).  The frame never
// moves during the pipelined pass, so the accumulators are never rescaled.  A
// score above m_ref + kFrameSlack (log2 units) sets ovf: the range is then
// redone, tile by tile without pipelining, with m_ref = the largest score of
// the whole range, which every column tracks.  Weights stay below
// 2^kFrameSlack in a pass that stands.
// ============================================================================
typedef __attribute__((ext_vector_type(16))) float v16f;
typedef __attribute__((ext_vector_type(4))) _Float16 half4;

constexpr int kBf16Threads = 512;

typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(16))) int i32x16;

// Tile sizes and operand types of the 8-wave kernel.
template <int D, bool I8>
struct MtCfg {
  static constexpr int KTB = I8 ? 64 * D : 128 * D;     // K tile bytes in the cache
  static constexpr int KTB_LDS = I8 ? KTB + 256 : KTB;  // + the tile's 64 key scales
  static constexpr int VTB = 128 * D;                    // V tile bytes (bf16)
  static constexpr int NQS = I8 ? D / 32 : D / 16;       // score k-steps
  using QOp = typename std::conditional<I8, i32x4, bf16x8>::type;
  // K(0), K(1), V(0), V(1), two 16 KiB weight-exchange buffers; Q staging
  // (f32, 512 D bytes) from K(1) on may need more
  static constexpr int LAYOUT = 2 * KTB_LDS + 2 * VTB + 2 * 16384;
  static constexpr int LDS = LAYOUT > KTB_LDS + 512 * D ? LAYOUT : KTB_LDS + 512 * D;
};

// Asynchronous copy of K tile kt into LDS: codes (and, I8, the tile's 64
// scales behind them) or bf16 values.
template <int D, bool I8, int NT = kBf16Threads>
__device__ __forceinline__ void load_k(const TileSrc& ksrc, const TileSrc& ssrc, int kt,
                                       unsigned char* dst, int w, int lane) {
  constexpr int KTB = MtCfg<D, I8>::KTB;
#pragma unroll
  for (int i = 0; i < (KTB + NT * 16 - 1) / (NT * 16); ++i) {
    const int off = (i * NT + w * 64) * 16;
    if (off < KTB) dma16(ksrc.rsrc, dst + off, kt * KTB + off + lane * 16);
  }
  if constexpr (I8)
    if (w == 0 && lane < 16) dma16(ssrc.rsrc, dst + KTB, kt * 256 + lane * 16);
}

// Both lane halves' values: lane l receives (x of lane l % 32, x of lane
// l % 32 + 32), with v_permlane32_swap (no LDS traffic).
__device__ __forceinline__ void halves(float x, float& lo, float& hi) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  lo = __uint_as_float(r[0]);
  hi = __uint_as_float(r[1]);
}

// An empty volatile asm that reads and writes x: code motion above the
// machine scheduler cannot move the computation of x past it, so each
// softmax slice stays in the chunk (between scheduling fences) it was
// written in instead of sinking to its first use.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  asm volatile("" : "+v"(x));
}

// A wave's column.
struct ColB {
  int lc, lh, m, lim;
  bool valid;
};

__device__ __forceinline__ ColB col_b(const Tiling& t, int cb, int start) {
  ColB c;
  c.lc = t.lane & 31;
  c.lh = t.lane >> 5;
  c.m = t.m_base + 32 * cb + c.lc;
  c.valid = c.m < t.M_total;
  c.lim = start + (c.valid ? c.m / t.G : 0);
  return c;
}

// Stationary Q^T operand, scaled by sl2e in f32 and rounded once to bf16.
// The workgroup's 128 columns of Q (f32, D values each) are first copied
// into LDS by the buffer-to-LDS DMA, every wave instruction moving one
// column's contiguous D * 4 bytes (D = 256) or several columns: column col's
// 16-byte chunk j (dims 4 j .. 4 j + 3) lands at granule
// col * D/4 + (j ^ (col mod D/4)).  The permutation costs nothing on the
// global side (a lane may fetch any address) and makes the operand reads of
// one k-step (32 columns, the same chunk of each) hit every LDS bank
// equally.  Columns past the chunk's end read the last valid column (their
// results are never stored).
template <int D>
__device__ __forceinline__ void dma_q(const Tiling& t, const float* __restrict__ q, int Hq,
                                      unsigned char* dst) {
  constexpr int NT = kBf16Threads, GR = D / 4;
  const int row_hi = min(t.R - 1, (t.m_base + kMTile - 1) / t.G);
  const float* base = q + ((size_t)t.row0 + t.row_lo) * Hq * D;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, (size_t)(row_hi - t.row_lo + 1) * Hq * D * 4);
  if constexpr (GR == kWave) {
    // one column per wave instruction (column 8 i + w): its (row, head), and
    // so the start of its D values, are the same for every lane of the wave
    // and are worked out once per instruction on the scalar unit
#pragma unroll
    for (int i = 0; i < kMTile * GR / NT; ++i) {
      const int col = __builtin_amdgcn_readfirstlane(i * (NT / GR) + t.w);
      const int m = min(t.m_base + col, t.M_total - 1);
      const int cbase = __builtin_amdgcn_readfirstlane(
          ((m / t.G - t.row_lo) * Hq + t.g * t.G + m % t.G) * D * 4);
      dma16(rs, dst + (size_t)(i * NT + t.w * 64) * 16, cbase + 16 * (t.lane ^ (col & (GR - 1))));
    }
  } else {
#pragma unroll
    for (int i = 0; i < kMTile * GR / NT; ++i) {
      const int p = i * NT + t.w * 64 + t.lane;  // LDS granule this lane fills
      const int col = p / GR, j = (p % GR) ^ (col & (GR - 1));
      const int m = min(t.m_base + col, t.M_total - 1);
      const int off = (((m / t.G - t.row_lo) * Hq + t.g * t.G + m % t.G) * D + 4 * j) * 4;
      dma16(rs, dst + (size_t)(i * NT + t.w * 64) * 16, off);
    }
  }
}

// This lane's operand registers from the staged Q: k-step ks holds dims
// 16 ks + 8 h .. 16 ks + 8 h + 7 of column 32 cb + lane % 32 (h = lane / 32).
template <int D>
__device__ __forceinline__ void take_q(const ColB& c, int cb, float sl2e,
                                       const float4* __restrict__ q_lds, bf16x8 (&qreg)[D / 16]) {
  constexpr int GR = D / 4;
  const int col = 32 * cb + c.lc, sw = col & (GR - 1);
  const float4* qc = q_lds + col * GR;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const int j = 4 * ks + 2 * c.lh;
    const float4 a = qc[j ^ sw];
    const float4 b = qc[(j + 1) ^ sw];
    float f[8];
    f[0] = a.x * sl2e; f[1] = a.y * sl2e; f[2] = a.z * sl2e; f[3] = a.w * sl2e;
    f[4] = b.x * sl2e; f[5] = b.y * sl2e; f[6] = b.z * sl2e; f[7] = b.w * sl2e;
    qreg[ks] = to_bf16x8(f);
  }
}

// Prepared Q (the fused append-and-prefill call): the append kernel has
// already multiplied each f32 Q value by scale * log2 e and rounded it to
// bf16 with the same converter take_q uses, into qb ([packed rows][Hq][D]
// bf16).  The M-tile's columns are staged as 16-byte granules of 8 dims, D / 8
// per column, granule j of column col at LDS granule col D/8 + (j ^ (col %
// (D/8))); a column past the chunk repeats the last one (its result is never
// stored).
template <int D>
__device__ __forceinline__ void dma_qb(const Tiling& t, const void* __restrict__ qb, int Hq,
                                       unsigned char* dst) {
  constexpr int NT = kBf16Threads, GR = D / 8;
  static_assert(kMTile * GR % NT == 0, "whole granules per thread");
  const int row_hi = min(t.R - 1, (t.m_base + kMTile - 1) / t.G);
  const unsigned char* base =
      static_cast<const unsigned char*>(qb) + ((size_t)t.row0 + t.row_lo) * Hq * D * 2;
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(base, (size_t)(row_hi - t.row_lo + 1) * Hq * D * 2);
#pragma unroll
  for (int i = 0; i < kMTile * GR / NT; ++i) {
    const int p = i * NT + t.w * 64 + t.lane;  // LDS granule this lane fills
    const int col = p / GR, j = (p % GR) ^ (col & (GR - 1));
    const int m = min(t.m_base + col, t.M_total - 1);
    const int off = (((m / t.G - t.row_lo) * Hq + t.g * t.G + m % t.G) * D + 8 * j) * 2;
    dma16(rs, dst + (size_t)(i * NT + t.w * 64) * 16, off);
  }
}

// The B operands of this lane's column from the staged granules: k-step ks
// takes dims 16 ks + 8 lh .. + 7, granule 2 ks + lh (as take_q).
template <int D>
__device__ __forceinline__ void take_qb(const ColB& c, int cb, const uint4* __restrict__ q_lds,
                                        bf16x8 (&qreg)[D / 16]) {
  constexpr int GR = D / 8;
  const int col = 32 * cb + c.lc, sw = col & (GR - 1);
  const uint4* qc = q_lds + col * GR;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) qreg[ks] = __builtin_bit_cast(bf16x8, qc[(2 * ks + c.lh) ^ sw]);
}

// int8 form: the column's symmetric codes (as the append quantises K rows)
// and sq = s_q * scale * log2 e.  Lane (l % 32, h) holds the 16 codes of dims
// 32 ks + 16 h .. 32 ks + 16 h + 15 for each k-step.  The amax covers the
// other half of the column through lane l ^ 32; a NaN or an infinity anywhere
// in the column makes its scale NaN (an infinity would give inf: either way
// the codes are 0 and every score of the column is NaN).  The two waves of a
// column block (kh = 0, 1) hold the same columns: each computes the codes of
// half the k-steps and they swap them through LDS, once every wave has read
// the f32 staging (two barriers; every thread of the block calls this).
template <int D>
__device__ __forceinline__ void take_q_i8(const ColB& c, int cb, int kh, int w, int lane,
                                          float sl2e, float4* __restrict__ q_lds,
                                          i32x4 (&qc)[D / 32], float& sq) {
  constexpr int GR = D / 4, NQS = D / 32, HALF = NQS / 2;
  const int col = 32 * cb + c.lc, sw = col & (GR - 1);
  const float4* qcol = q_lds + col * GR;
  float am = 0.f, nz = 0.f;  // max |x|; x * 0 summed (NaN once any x is NaN or infinite)
#pragma unroll
  for (int ks = 0; ks < NQS; ++ks)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 x = qcol[(8 * ks + 4 * c.lh + e) ^ sw];
      am = fmaxf(fmaxf(am, fabsf(x.x)), fmaxf(fabsf(x.y), fmaxf(fabsf(x.z), fabsf(x.w))));
      nz = fmaf(x.x, 0.f, fmaf(x.y, 0.f, fmaf(x.z, 0.f, fmaf(x.w, 0.f, nz))));
    }
  am = fmaxf(am, __shfl_xor(am, 32, kWave));
  nz += __shfl_xor(nz, 32, kWave);
  const float s = nz == nz ? am * kInv127 : __builtin_nanf("");
  const RowQuant rq(s);
  i32x4 own[HALF];
  bool ok = rq.fast;
#pragma unroll
  for (int j = 0; j < HALF; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float4 x = qcol[(8 * (kh * HALF + j) + 4 * c.lh + e) ^ sw];
      own[j][e] = (int)pack_codes4_fast(x.x, x.y, x.z, x.w, rq, ok);
    }
  if (__any(!ok)) {
#pragma unroll
    for (int j = 0; j < HALF; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float4 x = qcol[(8 * (kh * HALF + j) + 4 * c.lh + e) ^ sw];
        own[j][e] = (int)pack_codes4(x.x, x.y, x.z, x.w, rq);
      }
  }
  __syncthreads();  // the f32 staging is no longer read: it takes the codes
  i32x4* xc = reinterpret_cast<i32x4*>(q_lds);  // [wave][j][lane]
#pragma unroll
  for (int j = 0; j < HALF; ++j) xc[(w * HALF + j) * 64 + lane] = own[j];
  __syncthreads();
#pragma unroll
  for (int j = 0; j < HALF; ++j) {
    const i32x4 other = xc[((w ^ 4) * HALF + j) * 64 + lane];
    qc[j] = kh == 0 ? own[j] : other;
    qc[HALF + j] = kh == 0 ? other : own[j];
  }
  sq = s * sl2e;
}

// Operand indices (16-byte units) within a staged tile.
__device__ __forceinline__ int k_op_b(int ks, int kh, int lc, int lh) {
  return (2 * ks + lh) * 64 + 32 * kh + lc;
}
template <int D>
__device__ __forceinline__ int v_op_b(int db, int kb, int s, int lc, int lh) {
  return (kb * 4 + 2 * s + lh) * D + 32 * db + lc;
}
// Value chunk j (dim block j / 4 of this wave's half, key step j % 4; steps
// 0, 1 in this wave's own key half, 2, 3 in the partner's).
template <int D>
__device__ __forceinline__ int pv_op_b(int j, int kh, int lc, int lh) {
  const int kstep = j & 3;
  const int kb = (kstep >> 1) ? 1 - kh : kh;
  return v_op_b<D>(kh * (D / 64) + (j >> 2), kb, kstep & 1, lc, lh);
}

// Weight exchange slots (16-byte units): [parity][wave][s][lane].
__device__ __forceinline__ int xp_slot(int par, int w, int s, int lane) {
  return ((par * 8 + w) * 2 + s) * 64 + lane;
}

// One score k-step: s += K operand . Q operand (integer dots kept as bits).
template <bool I8, typename QOp>
__device__ __forceinline__ void score_mfma(v16f& s, uint4 kop, const QOp& qop) {
  if constexpr (I8)
    s = __builtin_bit_cast(v16f, __builtin_amdgcn_mfma_i32_32x32x32_i8(
                                     __builtin_bit_cast(i32x4, kop), qop,
                                     __builtin_bit_cast(i32x16, s), 0, 0, 0));
  else
    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, kop), qop, s, 0, 0, 0);
}

// int8: integer dots (bits in s) -> log2-domain scores dot * (sq * s_key), for
// the keys this lane holds (32 kh + 8 a + 4 h + e at register 4 a + e); the
// key scales follow the codes of the staged tile.
template <int D>
__device__ __forceinline__ void scale_scores(v16f& s, const uint4* __restrict__ k_lds, int kh,
                                             const ColB& c, float sq) {
  const float4* ks4 = reinterpret_cast<const float4*>(
      reinterpret_cast<const unsigned char*>(k_lds) + MtCfg<D, true>::KTB);
  const i32x16 si = __builtin_bit_cast(i32x16, s);
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const float4 k4 = ks4[8 * kh + 2 * a + c.lh];
    s[4 * a] = (float)si[4 * a] * (sq * k4.x);
    s[4 * a + 1] = (float)si[4 * a + 1] * (sq * k4.y);
    s[4 * a + 2] = (float)si[4 * a + 2] * (sq * k4.z);
    s[4 * a + 3] = (float)si[4 * a + 3] * (sq * k4.w);
  }
}

// Scores of one tile (this wave's key half), unpipelined.
template <int D, bool I8>
__device__ __forceinline__ void qk_tile_b(const uint4* __restrict__ k_lds,
                                          const typename MtCfg<D, I8>::QOp (&qreg)[MtCfg<D, I8>::NQS],
                                          v16f& s, int kh, const ColB& c, float sq) {
#pragma unroll
  for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
  for (int ks = 0; ks < MtCfg<D, I8>::NQS; ++ks)
    score_mfma<I8>(s, k_lds[k_op_b(ks, kh, c.lc, c.lh)], qreg[ks]);
  if constexpr (I8) scale_scores<D>(s, k_lds, kh, c, sq);
}

// Keys past the column's causal limit get -inf (tiles that cross a limit only).
__device__ __forceinline__ void mask_tile_b(v16f& s, int key0, const ColB& c) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
    s[i] = key0 + 8 * (i >> 2) + 4 * c.lh + (i & 3) > c.lim ? -INFINITY : s[i];
}

template <int D>
__device__ __forceinline__ void pv_chunk_b(int j, uint4 vop, const bf16x8 (&p_own)[2],
                                           const bf16x8 (&p_oth)[2], v16f (&acc)[D / 64]) {
  const int kstep = j & 3;
  acc[j >> 2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
      __builtin_bit_cast(bf16x8, vop), kstep < 2 ? p_own[kstep & 1] : p_oth[kstep & 1],
      acc[j >> 2], 0, 0, 0);
}

// One pipelined step (see above).  cur: scores of tile i (log2 domain, masked)
// in, weights out; p_cur: bf16 weights of tile i out; nxt: scores of tile i+1
// out; p_prev / p_oth: this wave's / the partner's bf16 weights of tile i-1,
// multiplied into acc with the V tile in v_lds (skipped when FIRST).
//
// Chunk c (c < NC = D/16) carries the score MFMA of k-step c, the value MFMA
// of chunk c, the LDS reads of a later chunk and softmax phase slices; a
// scheduling fence closes it.  A wave raises its issue priority for the
// chunk's LDS reads and MFMAs and lowers it again for the softmax slice.
// Without that the older of the two waves sharing a SIMD wins every MFMA
// slot both want, runs ahead and then waits at the next barrier while the
// younger one finishes the tile alone, one wave deep; with it the pair tends
// to alternate (one issuing MFMAs while the other runs its softmax slice).
//   phases: 0 max; 1 cross-half max, largest score and frame check;
//   2..9 exponentials (2 each); 10, 11 bf16 conversion of the weights;
//   12 running sum.
template <int D, bool FIRST, bool I8>
__device__ __forceinline__ void fused_step_b(const uint4* __restrict__ k_lds,
                                             const uint4* __restrict__ v_lds,
                                             const typename MtCfg<D, I8>::QOp (&qreg)[MtCfg<D, I8>::NQS],
                                             float sq, v16f& cur, v16f& nxt,
                                             const bf16x8 (&p_prev)[2], const bf16x8 (&p_oth)[2],
                                             bf16x8 (&p_cur)[2], v16f (&acc)[D / 64],
                                             const ColB& c, int kh, float m_use, float m_ref,
                                             float& m_all, float& l_run, bool& ovf) {
  constexpr int NC = D / 16;
  // operand reads run one chunk ahead (two for int8 K, whose score
  // k-steps span two chunks: measured 0.7% faster there, no change for bf16)
  constexpr int DIST = I8 ? 2 : 1;
  constexpr int NPH = 13;
#pragma unroll
  for (int i = 0; i < 16; ++i) nxt[i] = 0.f;
  float lmax = -INFINITY, ls = 0.f;
  // operand ring: [slot][0 K, 1 V]
  uint4 ring[DIST + 1][2];
  // I8: a score k-step covers two chunks (32 dims); it runs on even chunks
  auto issue = [&](int cc) {
    uint4(&r)[2] = ring[cc % (DIST + 1)];
    if (!I8 || (cc & 1) == 0) r[0] = k_lds[k_op_b(I8 ? cc / 2 : cc, kh, c.lc, c.lh)];
    if (!FIRST) r[1] = v_lds[pv_op_b<D>(cc, kh, c.lc, c.lh)];
  };
  auto phase = [&](int ph) {
    if (ph == 0) {
#pragma unroll
      for (int i = 0; i < 16; ++i) lmax = fmaxf(lmax, cur[i]);
      pin(lmax);
    } else if (ph == 1) {
      float lo, hi;
      halves(lmax, lo, hi);
      const float mx = fmaxf(lo, hi);
      m_all = fmaxf(m_all, mx);
      ovf = ovf || mx > m_ref + kFrameSlack;
    } else if (ph < 10) {
      const int i0 = (ph - 2) * 2;
#pragma unroll
      for (int i = i0; i < i0 + 2; ++i) {
        float pv = fast_exp2(cur[i] - m_use);
        pin(pv);
        cur[i] = pv;
        ls += pv;
      }
      pin(ls);
    } else if (ph < 12) {
      const int ss = ph - 10;
      float f[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) f[j] = cur[8 * ss + j];
      p_cur[ss] = to_bf16x8(f);
      pin(p_cur[ss]);
    } else {
      l_run += ls;
    }
  };

#pragma unroll
  for (int cc = 0; cc < DIST; ++cc) issue(cc);
#pragma unroll
  for (int cc = 0; cc < NC; ++cc) {
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    if (cc + DIST < NC) issue(cc + DIST);
    const uint4(&r)[2] = ring[cc % (DIST + 1)];
    if (!I8 || (cc & 1) == 0) score_mfma<I8>(nxt, r[0], qreg[I8 ? cc / 2 : cc]);
    if (!FIRST) pv_chunk_b<D>(cc, r[1], p_prev, p_oth, acc);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph)
      if (ph * NC / NPH == cc) phase(ph);
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (I8) scale_scores<D>(nxt, k_lds, kh, c, sq);
}

// 8-wave kernel: the flagged values of tile kt (see sanitize_tile), into the
// columns that see them.  xw: the tile's bf16 weights in exchange buffer 0
// (written by every wave; see fused_step_b for the slots), acc: dims
// kh D/2 + 32 db + 8 a + 4 h + 0..3 of the lane's column.
template <int D>
__device__ __forceinline__ void add_nonfinite_b(uint64_t nf, int kt, const uint4* __restrict__ xw,
                                                const uint32_t* __restrict__ tab, int cb, int kh,
                                                const ColB& c, v16f (&acc)[D / 64]) {
  uint32_t cls[D / 64];  // [db]: dims 32 db + 8 a + 4 h + e of this half at bits 2 (4 a + e)
#pragma unroll
  for (int db = 0; db < D / 64; ++db) cls[db] = 0u;
  while (nf != 0) {
    const int pl = __builtin_ctzll(nf);
    nf &= nf - 1;
    if (!c.valid || kt * kNTile + pl > c.lim) continue;
    // key pl of the tile: wave cb + 4 (pl / 32) holds it, in register 4 a + e
    // (k = pl % 32 = 8 a + 4 h + e) of lane lc + 32 h
    const int k = pl & 31;
    const uint4 wq = xw[xp_slot(0, cb + 4 * (pl >> 5), k >> 4, c.lc + 32 * ((k >> 2) & 1))];
    const int el = 4 * ((k >> 3) & 1) + (k & 3);
    const uint32_t word = (el >> 1) == 0 ? wq.x : (el >> 1) == 1 ? wq.y : (el >> 1) == 2 ? wq.z : wq.w;
    const bool zero_w = ((word >> (16 * (el & 1))) & 0x7fffu) == 0u;
#pragma unroll
    for (int db = 0; db < D / 64; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d0 = kh * (D / 2) + 32 * db + 8 * a + 4 * c.lh;
        uint32_t byte = (tab[pl * (D / 16) + d0 / 16] >> (2 * (d0 % 16))) & 0xffu;
        if (zero_w) byte = all_nan(byte);
        cls[db] |= byte << (8 * a);
      }
  }
#pragma unroll
  for (int db = 0; db < D / 64; ++db) apply_classes<16>(cls[db], acc[db], 0);
}

// Stores the workgroup's 128 columns: the normalised output (one split) or
// the split's partial.  Partials: acc [tile][S][128 columns][D] as binary16,
// each lane's D / 4 values scaled by 2^-e so that the largest finite one lies
// in [0.5, 1) (rounding adds at most 2^-12 of it); records (m, l, e of (half
// kh, lane half h) at 2 + 2 kh + h) [tile][128 columns][S][6].
//
// A lane holds 4-value pieces of its column spread over the column's dims, so
// the values go through LDS first: each wave writes its pieces into a
// [128 columns][D] staging array (from the start of the LDS, free by now) whose
// 16-byte granules are permuted within each column row (granule k of column
// col at position k ^ (col mod granules per row), which spreads the 32
// columns of one write over the LDS banks), and after a barrier every thread
// stores whole granules, so each wave instruction writes 1 KiB of
// consecutive bytes.  Every thread of the block calls this (it holds
// barriers); lanes of columns past the chunk's end store nothing.
template <int D>
__device__ __forceinline__ void store_result_b(const Tiling& t, const ColB& c, int kh,
                                               float* __restrict__ out, void* __restrict__ part,
                                               float* __restrict__ part_ml,
                                               const v16f (&acc)[D / 64], float m_ref, float l_tot,
                                               int Hq, int S, unsigned char* __restrict__ stage) {
  constexpr int NT = kBf16Threads;
  const int col = c.m - t.m_base;  // 0 .. 127
  __syncthreads();                 // every wave is done with the tiles and exchanges
  if (S == 1) {
    // f32 granules of 4 dims, D / 4 per column
    constexpr int GR = D / 4;
    float4* st = reinterpret_cast<float4*>(stage);
    const float sc = 1.f / l_tot;
    // lane holds dims 32 db + 8 a + 4 h + 0..3 of this wave's half
#pragma unroll
    for (int db = 0; db < D / 64; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int k = kh * (D / 8) + 8 * db + 2 * a + c.lh;
        st[col * GR + (k ^ (col & (GR - 1)))] =
            make_float4(acc[db][4 * a] * sc, acc[db][4 * a + 1] * sc, acc[db][4 * a + 2] * sc,
                        acc[db][4 * a + 3] * sc);
      }
    __syncthreads();
    for (int gi = t.tid; gi < kMTile * GR; gi += NT) {
      const int cc = gi / GR, k = gi - cc * GR, m = t.m_base + cc;
      if (m >= t.M_total) continue;
      float* op = out + (((size_t)t.row0 + m / t.G) * Hq + t.g * t.G + m % t.G) * D;
      reinterpret_cast<float4*>(op)[k] = st[cc * GR + (k ^ (cc & (GR - 1)))];
    }
    return;
  }
  float amax = 0.f;
#pragma unroll
  for (int db = 0; db < D / 64; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float x = fabsf(acc[db][i]);
      amax = x <= FLT_MAX ? fmaxf(amax, x) : amax;  // finite values only
    }
  int e = 0;
  if (amax > 0.f) (void)frexpf(amax, &e);
  const float sc = ldexpf(1.f, -e);
  // binary16 granules of 8 dims, D / 8 per column; a lane's 4 values are
  // half a granule
  constexpr int GR = D / 8;
  half4* st = reinterpret_cast<half4*>(stage);
#pragma unroll
  for (int db = 0; db < D / 64; ++db)
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      half4 h;
#pragma unroll
      for (int k = 0; k < 4; ++k) h[k] = (_Float16)(acc[db][4 * a + k] * sc);
      const int k = kh * (D / 16) + 4 * db + a;
      st[2 * (col * GR + (k ^ (col & (GR - 1)))) + c.lh] = h;
    }
  if (c.valid) {
    float* ml = part_ml + ((size_t)t.slot * kMTile + (size_t)col * S + t.split) * 6;
    if (kh == 0 && c.lh == 0) {
      ml[0] = m_ref;
      ml[1] = l_tot;
    }
    ml[2 + 2 * kh + c.lh] = (float)e;
  }
  __syncthreads();
  const uint4* sg = reinterpret_cast<const uint4*>(stage);
  uint4* pp = reinterpret_cast<uint4*>(reinterpret_cast<_Float16*>(part) +
                                       ((size_t)t.slot + t.split) * kMTile * D);
  for (int gi = t.tid; gi < kMTile * GR; gi += NT) {
    const int cc = gi / GR, k = gi - cc * GR;
    if (t.m_base + cc >= t.M_total) continue;
    pp[gi] = sg[cc * GR + (k ^ (cc & (GR - 1)))];
  }
}

// QB (bf16 caches): q points at prepared bf16 Q (see dma_qb) instead of f32.
template <int D, bool I8, bool QB = false>
__global__ __launch_bounds__(kBf16Threads) void prefill_mtile_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, void* __restrict__ part,
    float* __restrict__ part_ml, const float* __restrict__ k_scales, int Hq, int Hkv, int C,
    const ChunkArg ca, float sl2e) {
  using Cfg = MtCfg<D, I8>;
  constexpr int KTB = Cfg::KTB, KTB_LDS = Cfg::KTB_LDS, VTB = Cfg::VTB;
  constexpr int NT = kBf16Threads;
  // K(0), K(1), V(0), V(1), then two weight-exchange buffers of 16 KiB.  The
  // exchange buffer that holds no weights at that moment also carries the
  // per-pass exchanges (frame, votes, sums), so no other LDS is used:
  // 160 KiB at D = 256 for bf16 caches, 144.25 KiB for int8-K (whose Q
  // staging is larger than its tiles).
  __shared__ __attribute__((aligned(16))) unsigned char lds[Cfg::LDS];
  unsigned char* const kb0 = lds;
  unsigned char* const kb1 = lds + KTB_LDS;
  unsigned char* const vb0 = lds + 2 * KTB_LDS;
  unsigned char* const vb1 = vb0 + VTB;
  uint4* const xp = reinterpret_cast<uint4*>(vb1 + VTB);

  Tiling t;
  if (!make_tiling(ca, Hq, Hkv, t)) return;
  const int start = t.start, R = t.R, S = t.S;
  const int kh = t.w >> 2, partner = t.w ^ 4;
  const ColB c = col_b(t, t.w & 3, start);
  const size_t slab_i = (size_t)t.b * Hkv + t.g;
  const size_t k_slab = (size_t)C * D * (I8 ? 1 : 2);  // bytes
  const TileSrc ksrc = tile_src(reinterpret_cast<const unsigned char*>(k_cache) + slab_i * k_slab, k_slab);
  const TileSrc ssrc = tile_src(I8 ? k_scales + slab_i * C : nullptr, I8 ? (size_t)C * 4 : 0);
  const TileSrc vsrc = tile_src(reinterpret_cast<const unsigned char*>(v_cache) + slab_i * C * D * 2,
                                (size_t)C * D * 2);
  const unsigned char* v_slab_b = reinterpret_cast<const unsigned char*>(v_cache) + slab_i * C * D * 2;
  const int n = t.kt1 - t.kt0;
  const int vis_all = start + t.row_lo;  // positions every column of the tile sees

  typename Cfg::QOp qreg[Cfg::NQS];
  float sq = 0.f;  // I8: s_q * scale * log2 e of this lane's column
  v16f acc[D / 64];
  float m_ref = -INFINITY, m_all = -INFINITY, l_run = 0.f, l_tot = 0.f;
#pragma unroll
  for (int db = 0; db < D / 64; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;  // also the result of an empty split
  // Q (f32) is staged behind K(0): kb1 onwards, up to the end of the
  // exchange buffers (512 D bytes), which hold nothing until every wave has
  // taken its operands
  // Prepared bf16 Q takes half that, V(0) and V(1)'s buffers, so K(1) can
  // be fetched at once too.
  unsigned char* const q_lds = QB ? vb0 : kb1;
  static_assert(KTB_LDS + kMTile * D * 4 <= Cfg::LDS, "Q staging fits behind K(0)");
  static_assert(!QB || (!I8 && kMTile * D * 2 <= 2 * VTB), "bf16 Q fits the V buffers");
  if (n > 0) {
    load_k<D, I8>(ksrc, ssrc, t.kt0, kb0, t.w, t.lane);
    if constexpr (QB) {
      if (n > 1) load_k<D, I8>(ksrc, ssrc, t.kt0 + 1, kb1, t.w, t.lane);
      dma_qb<D>(t, q, Hq, q_lds);
    } else {
      dma_q<D>(t, q, Hq, q_lds);
    }
  }
  // per-pass exchange area (floats) in the exchange buffer that holds no
  // weights at that moment: [wave][slot][lane]
  auto xf = [&](int par, int w, int slot) {
    return reinterpret_cast<float*>(xp + xp_slot(par, 0, 0, 0)) + (w * 4 + slot) * 64 + t.lane;
  };

  v16f sa, sb;
  bf16x8 pw[2], pc[2], po[2];
  bool redo = false;

  // Pipelined pass in the frame of the first tile (see above).  A
  // non-finite V value that some column of a crossing tile cannot see (vbad)
  // also sends the range to the redo pass, which leaves it out of the shared
  // product (see nonfinite_v).
  if (n > 0) {
    bool ovf = false;
    wait_vmem();
    __syncthreads();  // K(0) and Q (QB: and K(1)) are in LDS
    if constexpr (QB) {
      // the V buffers are next written at the first step, after its barrier
      take_qb<D>(c, t.w & 3, reinterpret_cast<const uint4*>(q_lds), qreg);
    } else {
      if constexpr (I8)
        take_q_i8<D>(c, t.w & 3, kh, t.w, t.lane, sl2e, reinterpret_cast<float4*>(q_lds), qreg, sq);
      else
        take_q<D>(c, t.w & 3, sl2e, reinterpret_cast<const float4*>(q_lds), qreg);
      __syncthreads();  // every wave holds its Q: kb1 and the exchange buffers are free
      if (n > 1) load_k<D, I8>(ksrc, ssrc, t.kt0 + 1, kb1, t.w, t.lane);
    }
    // scores of the first tile (no softmax to overlap with yet)
    qk_tile_b<D, I8>(reinterpret_cast<const uint4*>(kb0), qreg, sa, kh, c, sq);
    if (t.kt0 * kNTile + kNTile - 1 > start + t.row_lo) mask_tile_b(sa, t.kt0 * kNTile + 32 * kh, c);
    {
      // frame: the first tile's largest score over both key halves; this
      // wave's half goes to exchange buffer 1 (first holds weights in step 1)
      float mx = -INFINITY, lo, hi;
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sa[i]);
      halves(mx, lo, hi);
      m_ref = fmaxf(lo, hi);
      *xf(1, t.w, 0) = m_ref;
    }
    float m_use = 0.f;

    // Step i (parity P = i & 1): K(i+1) and V(i-1) are in buffers 1-P; K(i+2)
    // and V(i) are loaded into buffers P, whose previous contents (K(i),
    // V(i-2)) every wave finished with in step i-1.  The weights of tile i go
    // to exchange buffer P (both waves of the pair read them back in step
    // i+1); those of tile i-1 are in buffer 1-P.
    auto step = [&](auto par, auto first, int i, v16f& cur, v16f& nxt) {
      constexpr int P = decltype(par)::value;
      constexpr bool FIRST = decltype(first)::value;
      const unsigned char* k_use = P == 0 ? kb1 : kb0;
      const unsigned char* v_use = P == 0 ? vb1 : vb0;
      unsigned char* k_load = P == 0 ? kb0 : kb1;
      unsigned char* v_load = P == 0 ? vb0 : vb1;
      const int kt = t.kt0 + i;
      wait_vmem();
      __syncthreads();
      wait_lgkm();
      // the older wave of each SIMD (waves 0-3) issues the tile copies: it
      // reaches the step barrier first (see fused_step_b)
      if (t.w < 4) {
        if (i + 2 < n) load_k<D, I8, NT / 2>(ksrc, ssrc, kt + 2, k_load, t.w, t.lane);
        load_tile<VTB, NT / 2>(vsrc, kt, v_load, t.w, t.lane);
      }
      if (FIRST) {
        m_ref = fmaxf(m_ref, *xf(1, partner, 0));
        m_use = m_ref == -INFINITY ? 0.f : m_ref;
        pin(m_use);
      } else {
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
          po[s2] = __builtin_bit_cast(bf16x8, xp[xp_slot(1 - P, partner, s2, t.lane)]);
        if (kt * kNTile + kNTile - 1 > start + t.row_lo) mask_tile_b(cur, kt * kNTile + 32 * kh, c);
      }
      fused_step_b<D, FIRST, I8>(reinterpret_cast<const uint4*>(k_use),
                                 reinterpret_cast<const uint4*>(v_use), qreg, sq, cur, nxt, pw, po,
                                 pc, acc, c, kh, m_use, m_ref, m_all, l_run, ovf);
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        xp[xp_slot(P, t.w, s2, t.lane)] = __builtin_bit_cast(uint4, pc[s2]);
        pw[s2] = pc[s2];  // this wave's own weights stay in registers
      }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    step(I0(), std::true_type(), 0, sa, sb);
    for (int i = 1; i < n; i += 2) {
      step(I1(), std::false_type(), i, sb, sa);
      if (i + 1 < n) step(I0(), std::false_type(), i + 1, sa, sb);
    }
    // value product of the last tile: V(n-1) in buffer (n-1) & 1, weights in
    // exchange buffer (n-1) & 1
    const int kt = t.kt1 - 1;
    const int pl = (n - 1) & 1;
    unsigned char* v_last = pl ? vb1 : vb0;
    wait_vmem();
    __syncthreads();
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
      po[s2] = __builtin_bit_cast(bf16x8, xp[xp_slot(pl, partner, s2, t.lane)]);
    if ((kt + 1) * kNTile > t.kend) {
      zero_v_beyond<D, true, NT>(reinterpret_cast<uint4*>(v_last), kt, t.kend, t.tid);
      __syncthreads();
    }
    // Crossing tiles are the last of the range: V(n-1) and V(n-2) are still
    // in LDS; an older one (an M-tile of more than 64 rows) is read again
    // from the cache.
    bool vbad = false;
    if (kt * kNTile + kNTile - 1 > vis_all)
      vbad = nonfinite_v<D, true, NT, false>(reinterpret_cast<uint4*>(v_last), kt, vis_all, t.kend,
                                             t.tid, nullptr) != 0;
    if (n > 1 && (kt - 1) * kNTile + kNTile - 1 > vis_all)
      vbad = vbad || nonfinite_v<D, true, NT, false>(reinterpret_cast<uint4*>(pl ? vb0 : vb1),
                                                     kt - 1, vis_all, t.kend, t.tid, nullptr) != 0;
    for (int k2 = kt - 2; k2 >= t.kt0 && k2 * kNTile + kNTile - 1 > vis_all; --k2)
      vbad = vbad || nonfinite_v<D, true, NT, false>(
                         const_cast<uint4*>(reinterpret_cast<const uint4*>(v_slab_b) + (size_t)k2 * (VTB / 16)),
                         k2, vis_all, t.kend, t.tid, nullptr) != 0;
    const uint4* vl = reinterpret_cast<const uint4*>(v_last);
#pragma unroll
    for (int j = 0; j < D / 16; ++j) pv_chunk_b<D>(j, vl[pv_op_b<D>(j, kh, c.lc, c.lh)], pw, po, acc);
    // votes, largest scores and sums, in exchange buffer 1 - pl (free since
    // the barrier above)
    const int px = 1 - pl;
    *xf(px, t.w, 1) = __any(ovf || vbad) ? 1.f : 0.f;
    *xf(px, t.w, 2) = m_all;
    *xf(px, t.w, 3) = l_run;
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < 8; ++w2) redo = redo || *xf(px, w2, 1) != 0.f;
    l_tot = l_run + *xf(px, partner, 3);
    if (redo) m_ref = fmaxf(m_all, *xf(px, partner, 2));
  }

  // Rare: a score left the frame, or a crossing tile holds a non-finite
  // value that some of its columns cannot see.  The range is redone, tile by
  // tile without pipelining, in the frame of its largest score, and such
  // values are left out of the shared product and added back where seen.
  if (redo) {
    // exchange buffer 1 (free until the sums below): the masks, then the
    // class table of a flagged tile (kNTile D / 4 bytes)
    uint32_t* const nfm = reinterpret_cast<uint32_t*>(xp + xp_slot(1, 0, 0, 0));
    uint32_t* const nf_tab = nfm + 64;
    static_assert(256 + kNTile * D / 4 <= 16384, "class table fits exchange buffer 1");
    l_run = 0.f;
#pragma unroll
    for (int db = 0; db < D / 64; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[db][i] = 0.f;
    const float m_use = m_ref == -INFINITY ? 0.f : m_ref;
    const uint4* kl = reinterpret_cast<const uint4*>(kb0);
    uint4* vl = reinterpret_cast<uint4*>(vb0);
    for (int i = 0; i < n; ++i) {
      const int kt = t.kt0 + i;
      __syncthreads();  // every wave is done with the previous tile and weights
      load_k<D, I8>(ksrc, ssrc, kt, kb0, t.w, t.lane);
      load_tile<VTB, NT>(vsrc, kt, vb0, t.w, t.lane);
      wait_vmem();
      __syncthreads();
      if ((kt + 1) * kNTile > t.kend) {
        zero_v_beyond<D, true, NT>(vl, kt, t.kend, t.tid);
        __syncthreads();
      }
      uint64_t nf = 0;
      if (kt * kNTile + kNTile - 1 > vis_all)
        nf = sanitize_tile<D, true, NT>(vl, kt, vis_all, t.kend, t.tid, nfm, nf_tab);
      v16f s;
      qk_tile_b<D, I8>(kl, qreg, s, kh, c, sq);
      if (kt * kNTile + kNTile - 1 > start + t.row_lo) mask_tile_b(s, kt * kNTile + 32 * kh, c);
      float ls = 0.f;
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        s[k] = fast_exp2(s[k] - m_use);
        ls += s[k];
      }
      l_run += ls;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        float f[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) f[j] = s[8 * s2 + j];
        pw[s2] = to_bf16x8(f);
        xp[xp_slot(0, t.w, s2, t.lane)] = __builtin_bit_cast(uint4, pw[s2]);
      }
      __syncthreads();
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2)
        po[s2] = __builtin_bit_cast(bf16x8, xp[xp_slot(0, partner, s2, t.lane)]);
#pragma unroll
      for (int j = 0; j < D / 16; ++j) pv_chunk_b<D>(j, vl[pv_op_b<D>(j, kh, c.lc, c.lh)], pw, po, acc);
      if (nf != 0) add_nonfinite_b<D>(nf, kt, xp, nf_tab, t.w & 3, kh, c, acc);
    }
    __syncthreads();
    *xf(1, t.w, 3) = l_run;
    __syncthreads();
    l_tot = l_run + *xf(1, partner, 3);
  }
  {
    float lo, hi;
    halves(l_tot, lo, hi);
    l_tot = lo + hi;
  }
  store_result_b<D>(t, c, kh, out, part, part_ml, acc, m_ref, l_tot, Hq, S, lds);
}

// Sequential prefill (one K+V stage) for shapes whose four tiles do not fit
// in LDS: copy tile i, then compute it, then copy tile i+1.
template <int D>
__global__ __launch_bounds__(256) void prefill_seq_kernel(
    const float* __restrict__ q, const void* __restrict__ k_cache,
    const void* __restrict__ v_cache, float* __restrict__ out, float* __restrict__ part,
    float* __restrict__ part_ml, int Hq, int Hkv, int C, const ChunkArg ca, float sl2e) {
  using Cfg = PrefillCfg<D, false>;
  constexpr int NDB = Cfg::NDB, TB = Cfg::TILE_BYTES;
  __shared__ __attribute__((aligned(16))) unsigned char kb[TB];
  __shared__ __attribute__((aligned(16))) unsigned char vb[TB];
  __shared__ uint32_t nfm[8];                  // non-finite value masks, [wave][2]
  __shared__ uint32_t nf_tab[kNTile * D / 16];  // and their classes

  Tiling t;
  if (!make_tiling(ca, Hq, Hkv, t)) return;
  const int start = t.start, R = t.R, m_tiles = t.m_tiles, S = t.S;
  const size_t slab = ((size_t)t.b * Hkv + t.g) * (size_t)C * D;
  const TileSrc ksrc = tile_src(reinterpret_cast<const unsigned char*>(k_cache) + slab * 4, (size_t)C * D * 4);
  const TileSrc vsrc = tile_src(reinterpret_cast<const unsigned char*>(v_cache) + slab * 4, (size_t)C * D * 4);

  v4f qreg[2][D / 16];
  load_q<D>(t, q, R, Hq, qreg);
  v4f acc_o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) acc_o[db][mb] = v4f{0.f, 0.f, 0.f, 0.f};
  float m_run[2] = {-INFINITY, -INFINITY};
  float l_run[2] = {0.f, 0.f};
  v4f sacc[4][2];
  for (int kt = t.kt0; kt < t.kt1; ++kt) {
    __syncthreads();  // every wave is done with the previous tile
    load_tile<TB>(ksrc, kt, kb, t.w, t.lane);
    load_tile<TB>(vsrc, kt, vb, t.w, t.lane);
    wait_vmem();
    __syncthreads();
    if ((kt + 1) * kNTile > t.kend) {
      zero_v_beyond<D, false>(reinterpret_cast<uint4*>(vb), kt, t.kend, t.tid);
      __syncthreads();
    }
    uint64_t nf = 0;
    if (kt * kNTile + kNTile - 1 > start + t.row_lo)  // crosses a row's limit
      nf = sanitize_tile<D, false, 256>(reinterpret_cast<uint4*>(vb), kt, start + t.row_lo,
                                        t.kend, t.tid, nfm, nf_tab);
    qk_tile<D>(reinterpret_cast<const uint4*>(kb), qreg, sacc, t.lr, t.lg);
    float alpha[2];
    softmax_tile(t, kt, start, sl2e, sacc, m_run, l_run, alpha);
    rescale_acc<NDB>(alpha, acc_o);
    pv_tile<D>(reinterpret_cast<const uint4*>(vb), sacc, acc_o, t.lr, t.lg);
    if (nf != 0) add_nonfinite_f32<D>(nf, kt, t, start, sacc, nf_tab, acc_o);
  }
  store_result<D>(t, out, part, part_ml, acc_o, m_run, l_run, R, Hq, Hkv, m_tiles, S);
}

// Merge of the split partials: two forms.  With few splits (S <= kMergeFew,
// the usual case for long chunks, whose many M-tiles fill the chip), thread
// (c, v) of a block owns column c of 16 and the float4 dims 4 v + 64 j of
// every split, and issues all its loads -- partials and (m, l, e) records --
// before it uses any, so it waits for memory once.  With more splits (few
// M-tiles over a long context), a block takes 4 columns x 64 dims and its
// four waves take every fourth split each, kMergeBatch loads in flight per
// lane and a running frame per wave, then combine through LDS.  Both sum in
// a fixed order, so results do not depend on timing.  H16: binary16 partials
// with per-lane exponents (the 8-wave kernel's format); otherwise f32 partials
// with (m, l) pairs.
constexpr int kMergeFew = 8;     // most splits of the column form
constexpr int kMergeGroups = 4;  // waves of the split form, each a subset of the splits
constexpr int kMergeBatch = 8;   // split loads in flight per lane (split form)

template <bool H16>
struct PartFmt {
  static constexpr int ML = H16 ? 6 : 2;  // floats per (column, split) record
};

template <int D, bool H16>
__device__ __forceinline__ float4 load_part(const void* base, size_t idx) {
  if constexpr (H16) {
    const half4 h = *reinterpret_cast<const half4*>(reinterpret_cast<const _Float16*>(base) + idx);
    return make_float4((float)h[0], (float)h[1], (float)h[2], (float)h[3]);
  } else {
    return *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(base) + idx);
  }
}

template <int D, bool H16>
__global__ __launch_bounds__(256) void prefill_merge_few_kernel(
    const void* __restrict__ part, const float* __restrict__ part_ml, float* __restrict__ out,
    int Hq, int Hkv, const ChunkArg ca) {
  constexpr int J = D / 64;
  constexpr int ML = PartFmt<H16>::ML;
  const int mt = blockIdx.x >> 3, cg = blockIdx.x & 7;
  const int g = blockIdx.y, i = blockIdx.z;  // KV head, session of the launch
  const int R = ca.rows[i], m_tiles = ca.m_tiles[i], S = ca.splits[i];
  if (mt >= m_tiles || S == 1) return;  // a single split wrote its output itself
  const size_t slot = (size_t)ca.slot0[i] + ((size_t)g * m_tiles + mt) * S;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x;
  const int c = tid >> 4, v = tid & 15;
  const int col = cg * 16 + c;
  const int m = mt * kMTile + col;
  if (m >= R * G) return;
  const float* ml = part_ml + (slot * kMTile + (size_t)col * S) * ML;
  const size_t pc = (slot * kMTile + col) * D + 4 * v;  // element index
  const size_t PS = (size_t)kMTile * D;                        // stride between splits
  float4 t[kMergeFew][J];
  float mv[kMergeFew], lv[kMergeFew], ev[kMergeFew][J];
#pragma unroll
  for (int k = 0; k < kMergeFew; ++k) {
    if (k < S) {
#pragma unroll
      for (int j = 0; j < J; ++j) t[k][j] = load_part<D, H16>(part, pc + k * PS + 64 * j);
      mv[k] = ml[ML * k];
      lv[k] = ml[ML * k + 1];
      // exponent of the lane that wrote dims 4 v + 64 j: half (4 v + 64 j) / (D / 2), lane half v & 1
#pragma unroll
      for (int j = 0; j < J; ++j)
        ev[k][j] = H16 ? ml[ML * k + 2 + 2 * ((4 * v + 64 * j) / (D / 2)) + (v & 1)] : 0.f;
    } else {
      mv[k] = -INFINITY;
      lv[k] = 0.f;
    }
  }
  float M = -INFINITY;
#pragma unroll
  for (int k = 0; k < kMergeFew; ++k) M = fmaxf(M, mv[k]);
  float4 a[J];
#pragma unroll
  for (int j = 0; j < J; ++j) a[j] = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int k = 0; k < kMergeFew; ++k) {
    // past S, or a split that saw none of the column's keys (a NaN sum, even
    // with m = -inf, still reaches the result)
    if (lv[k] == 0.f) continue;
    const float f = fast_exp2(mv[k] - M);
    L += f * lv[k];
#pragma unroll
    for (int j = 0; j < J; ++j) {
      const float w = H16 ? ldexpf(f, (int)ev[k][j]) : f;
      a[j].x += w * t[k][j].x; a[j].y += w * t[k][j].y; a[j].z += w * t[k][j].z; a[j].w += w * t[k][j].w;
    }
  }
  const float il = 1.f / L;
  const int row = m / G, hh = m % G;
  float* op = out + (((size_t)ca.row0[i] + row) * Hq + g * G + hh) * D + 4 * v;
#pragma unroll
  for (int j = 0; j < J; ++j)
    *reinterpret_cast<float4*>(op + 64 * j) =
        make_float4(a[j].x * il, a[j].y * il, a[j].z * il, a[j].w * il);
}

template <int D, bool H16>
__global__ __launch_bounds__(256) void prefill_merge_split_kernel(
    const void* __restrict__ part, const float* __restrict__ part_ml, float* __restrict__ out,
    int Hq, int Hkv, const ChunkArg ca) {
  constexpr int J = D / 64;
  constexpr int ML = PartFmt<H16>::ML;
  __shared__ float4 red[kMergeGroups][4][16];
  __shared__ float red_m[kMergeGroups][4], red_l[kMergeGroups][4];
  const int js = blockIdx.x % J, cq = (blockIdx.x / J) & 31, mt = (blockIdx.x / J) >> 5;
  const int g = blockIdx.y, i = blockIdx.z;  // KV head, session of the launch
  const int R = ca.rows[i], m_tiles = ca.m_tiles[i], S = ca.splits[i];
  if (mt >= m_tiles || S == 1) return;  // block-uniform: before any barrier
  const size_t slot = (size_t)ca.slot0[i] + ((size_t)g * m_tiles + mt) * S;
  const int G = Hq / Hkv;
  const int tid = threadIdx.x, sg = tid >> 6, c = (tid >> 4) & 3, v = tid & 15;
  const int col = cq * 4 + c;
  const int m = mt * kMTile + col;
  const bool valid = m < R * G;
  const int d = 64 * js + 4 * v;
  const float* ml = part_ml + (slot * kMTile + (size_t)col * S) * ML;
  const size_t pc = (slot * kMTile + col) * D + d;  // element index
  const size_t PS = (size_t)kMTile * D;                    // stride between splits
  // exponent slot of the lane that wrote these dims: half d / (D / 2), lane half v & 1
  const int eo = 2 + 2 * (d / (D / 2)) + (v & 1);
  float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
  float mw = -INFINITY, lw = 0.f;
  if (valid) {
    for (int s0 = sg; s0 < S; s0 += kMergeGroups * kMergeBatch) {
      float4 t[kMergeBatch];
      float mv[kMergeBatch], lv[kMergeBatch], ev[kMergeBatch];
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        const int s = s0 + kMergeGroups * k;
        if (s < S) {
          t[k] = load_part<D, H16>(part, pc + s * PS);
          mv[k] = ml[ML * s];
          lv[k] = ml[ML * s + 1];
          ev[k] = H16 ? ml[ML * s + eo] : 0.f;
        } else {
          t[k] = make_float4(0.f, 0.f, 0.f, 0.f);
          mv[k] = -INFINITY;
          lv[k] = 0.f;
          ev[k] = 0.f;
        }
      }
      float mb = mw;
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) mb = fmaxf(mb, mv[k]);
      if (mb > mw) {  // move the frame (mw = -inf: nothing added yet, factor 0)
        const float r = fast_exp2(mw - mb);
        a.x *= r; a.y *= r; a.z *= r; a.w *= r;
        lw *= r;
        mw = mb;
      }
#pragma unroll
      for (int k = 0; k < kMergeBatch; ++k) {
        if (lv[k] != 0.f) {  // a split that saw none of the column's keys adds nothing
          float f = fast_exp2(mv[k] - mw);
          lw += f * lv[k];
          if constexpr (H16) f = ldexpf(f, (int)ev[k]);
          a.x += f * t[k].x; a.y += f * t[k].y; a.z += f * t[k].z; a.w += f * t[k].w;
        }
      }
    }
  }
  red[sg][c][v] = a;
  if (v == 0) {
    red_m[sg][c] = mw;
    red_l[sg][c] = lw;
  }
  __syncthreads();
  if (sg != 0 || !valid) return;
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < kMergeGroups; ++w) M = fmaxf(M, red_m[w][c]);
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  float L = 0.f;
#pragma unroll
  for (int w = 0; w < kMergeGroups; ++w) {
    if (red_l[w][c] == 0.f) continue;
    const float f = fast_exp2(red_m[w][c] - M);
    const float4 x = red[w][c][v];
    o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
    L += f * red_l[w][c];
  }
  const float il = 1.f / L;
  const int row = m / G, hh = m % G;
  *reinterpret_cast<float4*>(out + (((size_t)ca.row0[i] + row) * Hq + g * G + hh) * D + d) =
      make_float4(o.x * il, o.y * il, o.z * il, o.w * il);
}

// Split count of a chunk: the one that minimises a model of the launch time.
// A workgroup's LDS tiles fill most of a CU's 160 KiB, so one runs per CU:
// ceil(workgroups / 256) rounds run back to back, each as long as its
// longest workgroup (fixed cost + its key tiles); splitting also costs the
// merge pass, which reads back the partials.  At most about three rounds of
// workgroups are considered, which bounds the workspace.  Times in ns.
constexpr int kCUs = 256;
constexpr int kMaxWgRounds = 3;

int max_splits(long long units) {
  const long long cap = (kMaxWgRounds * (long long)kCUs + units - 1) / units;
  return (int)(cap < kMaxSplits ? cap : kMaxSplits);
}

// units: the (KV head, m-tile) pairs of every session in the launch; nkt:
// this session's key tiles.
int choose_splits(const Shape& s, long long units, int nkt) {
  const double scale_d = s.head_dim / 256.0;
  const double tile_ns = (s.kv_dtype == kF32 ? 9000.0 : 1300.0) * scale_d;
  const double wg_ns = 3000.0, merge_ns = 4000.0, part_ns = 26.0 * scale_d;
  const int smax = max_splits(units);
  int best = 1;
  double best_t = 0.0;
  for (int S = 1; S <= smax && S <= nkt; ++S) {
    const long long wgs = units * S;
    const long long rounds = (wgs + kCUs - 1) / kCUs;
    const double t = rounds * (wg_ns + tile_ns * ((nkt + S - 1) / S)) +
                     (S > 1 ? merge_ns + part_ns * (double)wgs : 0.0);
    if (S == 1 || t < best_t * 0.999) {
      best_t = t;
      best = S;
    }
  }
  return best;
}

// One launch: its session table, and the largest m-tile and split counts
// among its sessions (the merge grid's extent and form).
struct ChunkLaunch {
  ChunkArg ca;
  int max_m, max_s;
};

// qb (bf16 caches only, may be null): Q prepared by the fused append (see
// dma_qb), read in place of q.
template <int D, int MODE>
hipError_t launch_chunks(const Shape& s, const ChunkLaunch* L, int nl, long long total_slots,
                         const float* q, const void* kc, const void* vc, float* out, float scale,
                         void* ws, hipStream_t st, const void* qb = nullptr) {
  constexpr bool H16 = MODE != kF32;  // binary16 partials (the 8-wave kernel)
  using Cfg = PrefillCfg<D, false>;
  // partials: binary16 accumulators for bf16 and int8-K caches, f32 otherwise, one
  // 128-column slot per (session, KV head, m-tile, split); then the
  // per-(column, split) records
  float* part = reinterpret_cast<float*>(ws);
  float* part_ml = reinterpret_cast<float*>(reinterpret_cast<unsigned char*>(ws) +
                                            (size_t)total_slots * kMTile * D * (H16 ? 2 : 4));
  for (int l = 0; l < nl; ++l) {
    const ChunkArg& ca = L[l].ca;
    const int items = ca.item0[ca.n];
    if (items == 0) continue;
    // padded to whole rounds of the 8 XCDs (see make_tiling)
    const dim3 grid(8 * ((items + 7) / 8));
    if constexpr (MODE == kBF16) {
      if (qb)
        hipLaunchKernelGGL((prefill_mtile_kernel<D, false, true>), grid, dim3(kBf16Threads), 0, st,
                           static_cast<const float*>(qb), kc, vc, out, part, part_ml, nullptr,
                           s.num_q_heads, s.num_kv_heads, s.capacity, ca, scale * kLog2e);
      else
        hipLaunchKernelGGL((prefill_mtile_kernel<D, false>), grid, dim3(kBf16Threads), 0, st, q,
                           kc, vc, out, part, part_ml, nullptr, s.num_q_heads, s.num_kv_heads,
                           s.capacity, ca, scale * kLog2e);
    }
    else if constexpr (MODE == kI8K)
      hipLaunchKernelGGL((prefill_mtile_kernel<D, true>), grid, dim3(kBf16Threads), 0, st, q, kc,
                         vc, out, part, part_ml, k_scale_array(s, kc), s.num_q_heads,
                         s.num_kv_heads, s.capacity, ca, scale * kLog2e);
    else if constexpr (Cfg::PIPE)
      hipLaunchKernelGGL((prefill_pipe_kernel<D>), grid, dim3(256), 0, st, q, kc, vc, out,
                         part, part_ml, s.num_q_heads, s.num_kv_heads, s.capacity, ca,
                         scale * kLog2e);
    else
      hipLaunchKernelGGL((prefill_seq_kernel<D>), grid, dim3(256), 0, st, q, kc, vc, out,
                         part, part_ml, s.num_q_heads, s.num_kv_heads, s.capacity, ca,
                         scale * kLog2e);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (L[l].max_s > 1) {
      if (L[l].max_s <= kMergeFew)
        hipLaunchKernelGGL((prefill_merge_few_kernel<D, H16>),
                           dim3(L[l].max_m * (kMTile / 16), s.num_kv_heads, ca.n), dim3(256), 0, st,
                           part, part_ml, out, s.num_q_heads, s.num_kv_heads, ca);
      else
        hipLaunchKernelGGL((prefill_merge_split_kernel<D, H16>),
                           dim3(L[l].max_m * (kMTile / 4) * (D / 64), s.num_kv_heads, ca.n),
                           dim3(256), 0, st, part, part_ml, out, s.num_q_heads, s.num_kv_heads, ca);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

// Session tables of a call: the sessions with rows, kChunkSessions per
// launch, packed rows in session order, partial slots numbered across the
// whole call.  rows_of(b) / start_of(b): session b's chunk; splits_of(b, m):
// its split count given its m-tile count.  Returns the call's slot count.
template <class Rows, class Start, class Splits>
long long build_launches(const Shape& s, Rows rows_of, Start start_of, Splits splits_of,
                         std::vector<ChunkLaunch>& out) {
  const int G = s.num_q_heads / s.num_kv_heads;
  long long slot = 0, row = 0;
  ChunkLaunch cur{};
  for (int b = 0; b < s.batch; ++b) {
    const int R = rows_of(b);
    if (R <= 0) continue;
    if (cur.ca.n == kChunkSessions) {
      out.push_back(cur);
      cur = ChunkLaunch{};
    }
    ChunkArg& ca = cur.ca;
    const int i = ca.n;
    const int m = (int)(((long long)R * G + kMTile - 1) / kMTile);
    const int S = splits_of(b, m);
    ca.b[i] = b;
    ca.start[i] = start_of(b);
    ca.rows[i] = R;
    ca.m_tiles[i] = m;
    ca.splits[i] = S;
    ca.row0[i] = (int)row;
    ca.slot0[i] = (int)slot;
    ca.item0[i + 1] = ca.item0[i] + s.num_kv_heads * m * S;
    ca.n = i + 1;
    if (m > cur.max_m) cur.max_m = m;
    if (S > cur.max_s) cur.max_s = S;
    row += R;
    slot += (long long)s.num_kv_heads * m * S;
  }
  if (cur.ca.n > 0) out.push_back(cur);
  return slot;
}

template <int D>
hipError_t launch_mode(const Shape& s, const std::vector<ChunkLaunch>& L, long long slots,
                       const float* q, const void* kc, const void* vc, float* out, float scale,
                       void* ws, hipStream_t st, const void* qb = nullptr) {
  const int n = (int)L.size();
  switch (s.kv_dtype) {
    case kBF16: return launch_chunks<D, kBF16>(s, L.data(), n, slots, q, kc, vc, out, scale, ws, st, qb);
    case kI8K: return launch_chunks<D, kI8K>(s, L.data(), n, slots, q, kc, vc, out, scale, ws, st);
    default: return launch_chunks<D, kF32>(s, L.data(), n, slots, q, kc, vc, out, scale, ws, st);
  }
}

template <int D>
hipError_t launch_t(const Shape& s, const PrefillPlan& p, const float* q, const void* kc,
                    const void* vc, float* out, int start, int R, float scale, void* ws,
                    hipStream_t st, const void* qb) {
  std::vector<ChunkLaunch> L;
  const long long slots = build_launches(
      s, [&](int) { return R; }, [&](int) { return start; }, [&](int, int) { return p.splits; }, L);
  return launch_mode<D>(s, L, slots, q, kc, vc, out, scale, ws, st, qb);
}

}  // namespace

// Workspace bytes per (column, split): binary16 accumulators and a 6-float
// record for bf16 and int8-K caches, f32 accumulators and an (m, l) pair
// otherwise.
static size_t partial_bytes(const Shape& s) {
  return s.kv_dtype != kF32 ? (size_t)s.head_dim * 2 + 6 * sizeof(float)
                            : (size_t)(s.head_dim + 2) * sizeof(float);
}

// Chunks of at most kRowsMaxRows rows on bf16 caches may go to the streaming
// decode kernel, its columns taken by the chunk's (row, head) pairs: it reads
// each K / V row once per group of 16 pairs (the head groups of a split share
// an XCD's L2, so the groups after the first mostly hit there), while an
// M-tile spends the MFMA and LDS work of 128 columns whatever number of them
// is used.  The faster one is picked on two estimates, in ns, linear in the
// K / V positions read (sessions x KV heads x context) -- fits to measured
// times on 8 query heads per KV head, head_dim 256, contexts 1K .. 128K,
// batches 1 and 4: the streaming kernel's cost per position grows with its
// head groups; the M-tile path pays about twice as much per position when
// there is a single M-tile to split (all its parallelism then comes from
// splitting the context) than when there are several, plus a cost per row.
constexpr int kRowsMaxRows = 15;
constexpr int kRowsMaxGroups = 8;

static int rows_groups(const Shape& s, int R) {
  const int G = s.num_q_heads / s.num_kv_heads;
  return (R * G + 15) / 16;
}

static bool rows_path(const Shape& s, int R, int ctx) {
  if (s.kv_dtype == kF32 || R > kRowsMaxRows) return false;
  const int G = s.num_q_heads / s.num_kv_heads;
  const int hg = rows_groups(s, R);
  if (hg > kRowsMaxGroups) return false;
  const double pos = (double)s.batch * s.num_kv_heads * ctx * (s.head_dim / 256.0);
  const long long units = (long long)s.batch * s.num_kv_heads * ((R * G + kMTile - 1) / kMTile);
  const double t_rows = 10500.0 + pos * (0.17 + 0.06 * (hg - 1));
  const double t_tile = 14000.0 + 350.0 * R + pos * (units == 1 ? 0.36 : 0.18);
  return t_rows <= t_tile;
}

PrefillPlan plan_prefill(const Shape& s, int start, int R) {
  PrefillPlan p{};
  if (rows_path(s, R, start + R)) {
    p.m_tiles = 0;
    p.rows = plan_rows(s, R, start + R);
    p.splits = p.rows.splits;
    p.workspace_bytes = p.rows.workspace_bytes;
    return p;
  }
  const int G = s.num_q_heads / s.num_kv_heads;
  const long long M = (long long)R * G;
  p.m_tiles = (int)((M + kMTile - 1) / kMTile);
  const int nkt = (start + R - 1) / kNTile + 1;
  p.splits = choose_splits(s, (long long)s.batch * s.num_kv_heads * p.m_tiles, nkt);
  p.workspace_bytes = p.splits == 1 ? 0
      : (size_t)s.batch * s.num_kv_heads * p.m_tiles * p.splits * kMTile * partial_bytes(s);
  return p;
}

size_t prefill_workspace_bound(const Shape& s, int max_rows) {
  if (max_rows <= 0) return 0;
  if (max_rows > s.capacity) max_rows = s.capacity;  // no chunk holds more rows
  const int G = s.num_q_heads / s.num_kv_heads;
  const int mt_max = (int)(((long long)max_rows * G + kMTile - 1) / kMTile);
  size_t best = 0;
  for (int mt = 1; mt <= mt_max; ++mt) {
    const long long units = (long long)s.batch * s.num_kv_heads * mt;
    if (units >= (long long)kMaxWgRounds * kCUs) break;  // from here on no chunk splits
    const int S = max_splits(units);  // choose_splits never exceeds it
    if (S <= 1) continue;
    const size_t bytes = (size_t)units * S * kMTile * partial_bytes(s);
    if (bytes > best) best = bytes;
  }
  // few-row chunks that may take the streaming kernel: its split count
  // grows with the context, so the full capacity bounds every start
  for (int R = 1; R <= max_rows && R <= kRowsMaxRows; ++R) {
    if (s.kv_dtype == kF32 || rows_groups(s, R) > kRowsMaxGroups) break;
    const size_t bytes = plan_rows(s, R, s.capacity).workspace_bytes;
    if (bytes > best) best = bytes;
  }
  return best;
}

// Ragged calls: each session's split count is the one a uniform chunk of its
// own length would get with the call's total m-tile count.
static long long ragged_launches(const Shape& s, const int32_t* start, const int32_t* rows,
                                 std::vector<ChunkLaunch>& L) {
  const int G = s.num_q_heads / s.num_kv_heads;
  long long units = 0;
  for (int b = 0; b < s.batch; ++b)
    if (rows[b] > 0) units += (long long)s.num_kv_heads * (((long long)rows[b] * G + kMTile - 1) / kMTile);
  return build_launches(
      s, [&](int b) { return rows[b]; }, [&](int b) { return start[b]; },
      [&](int b, int) { return choose_splits(s, units, (start[b] + rows[b] - 1) / kNTile + 1); }, L);
}

size_t prefill_ragged_workspace(const Shape& s, const int32_t* start, const int32_t* rows) {
  std::vector<ChunkLaunch> L;
  const long long slots = ragged_launches(s, start, rows, L);
  bool split = false;
  for (const ChunkLaunch& l : L) split = split || l.max_s > 1;
  return split ? (size_t)slots * kMTile * partial_bytes(s) : 0;
}

// Every session's split count is at most max_splits(U) for the call's total
// m-tile count U, so the slots number at most U max_splits(U); U is at most
// Hkv (ceil(T G / 128) + min(B, T)) for T rows in all.
size_t prefill_ragged_workspace_bound(const Shape& s, long long max_total_rows) {
  if (max_total_rows <= 0) return 0;
  // no valid call holds more rows than every session's full capacity
  if (max_total_rows > (long long)s.batch * s.capacity) max_total_rows = (long long)s.batch * s.capacity;
  const int G = s.num_q_heads / s.num_kv_heads;
  const long long sessions = max_total_rows < s.batch ? max_total_rows : s.batch;
  const long long u_max = (long long)s.num_kv_heads * ((max_total_rows * G + kMTile - 1) / kMTile + sessions);
  long long most = 0;
  // past kMaxWgRounds * kCUs units no session splits and nothing is stored
  for (long long u = 1; u <= u_max && u <= (long long)kMaxWgRounds * kCUs; ++u) {
    const int S = max_splits(u);
    if (S > 1 && u * S > most) most = u * S;
  }
  return (size_t)most * kMTile * partial_bytes(s);
}

hipError_t launch_prefill_ragged(const Shape& s, const float* q, const void* k_cache,
                                 const void* v_cache, float* out, const int32_t* start,
                                 const int32_t* rows, float scale, void* workspace,
                                 hipStream_t stream) {
  std::vector<ChunkLaunch> L;
  const long long slots = ragged_launches(s, start, rows, L);
  switch (s.head_dim) {
    case 64: return launch_mode<64>(s, L, slots, q, k_cache, v_cache, out, scale, workspace, stream);
    case 128: return launch_mode<128>(s, L, slots, q, k_cache, v_cache, out, scale, workspace, stream);
    case 256: return launch_mode<256>(s, L, slots, q, k_cache, v_cache, out, scale, workspace, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill(const Shape& s, const PrefillPlan& p, const float* q,
                          const void* k_cache, const void* v_cache, float* out, int start, int R,
                          float scale, void* workspace, hipStream_t stream, const void* qb) {
  if (p.m_tiles == 0)
    return launch_rows(s, p.rows, q, k_cache, v_cache, out, start, R, scale, workspace, stream);
  if (qb && s.kv_dtype != kBF16) return hipErrorInvalidValue;
  switch (s.head_dim) {
    case 64: return launch_t<64>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream, qb);
    case 128: return launch_t<128>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream, qb);
    case 256: return launch_t<256>(s, p, q, k_cache, v_cache, out, start, R, scale, workspace, stream, qb);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace ka
