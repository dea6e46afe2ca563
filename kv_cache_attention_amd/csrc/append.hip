// KV append: new f32 rows [rows][Hkv][D] of each session -> its cache
// positions start .. start + rows - 1 (a uniform chunk: every session the
// same start and rows, rows packed session by session as [B][R][Hkv][D]).
//
// One thread produces one 16-byte cache vector, so every store is a full
// 16-byte store except where a V vector (which spans 4 or 8 positions) is
// only partly covered by the appended range; there the covered elements are
// stored one by one and the rest of the vector is left untouched.
#include <vector>

#include "ka_common.h"
#include "ka_launch.h"

namespace ka {

// Rotary embedding of element d of a row x (rotate-half pairing: dims d and
// d + D/2 form one pair, turned by the angle whose cos / sin are c[d mod D/2],
// s[d mod D/2]).  Two rounded products and one rounded sum or difference, in
// that order: no fused multiply-add, so the result is reproducible bit for
// bit.
// A product held opaque to the code generator, so it cannot be fused into a
// multiply-add with the sum that follows (the library builds with FP
// contraction on).
__device__ __forceinline__ float rounded_mul(float a, float b) {
  float p = a * b;
  asm volatile("" : "+v"(p));
  return p;
}

// Four pairs at once: a = x[j .. j+3], b = x[j+D/2 .. j+D/2+3], c / s the
// row's cos / sin at j .. j+3.  lo gets the first-half outputs, hi the second.
__device__ __forceinline__ void rope4(float4 a, float4 b, float4 c, float4 s, float4& lo,
                                      float4& hi) {
  lo.x = rounded_mul(a.x, c.x) - rounded_mul(b.x, s.x);
  lo.y = rounded_mul(a.y, c.y) - rounded_mul(b.y, s.y);
  lo.z = rounded_mul(a.z, c.z) - rounded_mul(b.z, s.z);
  lo.w = rounded_mul(a.w, c.w) - rounded_mul(b.w, s.w);
  hi.x = rounded_mul(b.x, c.x) + rounded_mul(a.x, s.x);
  hi.y = rounded_mul(b.y, c.y) + rounded_mul(a.y, s.y);
  hi.z = rounded_mul(b.z, c.z) + rounded_mul(a.z, s.z);
  hi.w = rounded_mul(b.w, c.w) + rounded_mul(a.w, s.w);
}

// The sessions of one append launch, one per blockIdx.y: session i writes
// rows[i] rows at positions start[i] .. of cache slab b[i], reading rows
// row0[i] .. of k_new / v_new and cos / sin rows rope_row0[i] ...
constexpr int kAppendSessions = 32;
struct AppendArg {
  int n;
  int b[kAppendSessions], start[kAppendSessions], rows[kAppendSessions];
  int row0[kAppendSessions], rope_row0[kAppendSessions];
};

// First V group and group count overlapping positions [start, start + R)
// (a group holds E positions; bf16 groups interleave within a 32-position
// block, so whole blocks are covered).
__host__ __device__ __forceinline__ void v_groups(bool bf16, int start, int R, int& g0, int& ng) {
  int g1;
  if (bf16) {
    g0 = (start >> 5) * 4;
    g1 = ((start + R - 1) >> 5) * 4 + 4;
  } else {
    g0 = start >> 2;
    g1 = ((start + R - 1) >> 2) + 1;
  }
  ng = g1 - g0;
}

// Dims d .. d + 3 (d a multiple of 4) of a K row as stored: as given, or
// rotated (rotate-half pairs) with the row's cos / sin rows cr / sr.
template <bool ROPE>
__device__ __forceinline__ float4 k_dims4(const float* rowp, const float* cr, const float* sr,
                                          int d, int D) {
  if constexpr (!ROPE) {
    return *reinterpret_cast<const float4*>(rowp + d);
  } else {
    const int h = D >> 1, j = d < h ? d : d - h;
    float4 lo, hi;
    rope4(*reinterpret_cast<const float4*>(rowp + j), *reinterpret_cast<const float4*>(rowp + j + h),
          *reinterpret_cast<const float4*>(cr + j), *reinterpret_cast<const float4*>(sr + j), lo, hi);
    return d < h ? lo : hi;
  }
}

// int8 K: one wave quantises one row.  Lane l takes dims 4 l .. 4 l + 3
// (lanes past D / 4 take none), the amax and the NaN flag are reduced across
// the wave, and every lane stores its four codes as one 32-bit word of the
// row's 16-byte code vectors; lane 0 stores the scale.  codes: the slab's
// code bytes; vec_base(c): the byte offset of the row's code vector c.
template <bool ROPE>
__device__ __forceinline__ void quantise_row_wave(const float* rowp, const float* cr,
                                                  const float* sr, int D, int lane,
                                                  int8_t* codes, size_t row_vec0, float* scale_out) {
  const bool mine = 4 * lane < D;
  const float4 x = mine ? k_dims4<ROPE>(rowp, cr, sr, 4 * lane, D) : make_float4(0.f, 0.f, 0.f, 0.f);
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
  const float s = row.scale();
  if (mine) {
    // dims 4 l .. 4 l + 3 sit in code vector l / 4, bytes 4 (l % 4) .. + 3; vectors
    // of one row are 64 vectors (1 KiB) apart in the [D/16][64][16] block layout
    const size_t off = (row_vec0 + (size_t)(lane >> 2) * 64) * 16 + 4 * (lane & 3);
    const RowQuant rq(s);
    bool ok = rq.fast;
    uint32_t wc = pack_codes4_fast(x.x, x.y, x.z, x.w, rq, ok);
    if (__any(!ok)) wc = pack_codes4(x.x, x.y, x.z, x.w, rq);
    *reinterpret_cast<uint32_t*>(codes + off) = wc;
  }
  if (lane == 0) *scale_out = s;
}

// ROPE: each new K row is rotated by its position's angles (cos / sin rows of
// D/2 values, one per appended row) before it is stored; V as given.  MODE
// (KvMode): f32 K / V; bf16 K / V; int8 K codes with their row scales in
// k_scales ([B][Hkv][C] f32) and bf16 V.  QB (bf16, for the fused append and
// prefill): the chunk's Q rows q ([rows][Hq][D] f32, packed like k_new) also
// go to qb as bf16 of q * sl2e, with the rounding the prefill kernel applies
// to its Q operands, 8 dims per 16-byte vector.
template <int MODE, bool ROPE, bool QB = false>
__global__ __launch_bounds__(256) void append_kernel(
    void* __restrict__ k_cache, void* __restrict__ v_cache,
    const float* __restrict__ k_new, const float* __restrict__ v_new,
    const float* __restrict__ rope_cos, const float* __restrict__ rope_sin,
    float* __restrict__ k_scales, int Hkv, int D, int C, const AppendArg aa,
    const float* __restrict__ q, uint4* __restrict__ qb, int Hq, float sl2e) {
  static_assert(!QB || MODE == kBF16, "prepared Q only with bf16 caches");
  constexpr bool BF16 = MODE != kF32;             // V (and bf16 K) in the bf16 layouts
  constexpr int E = BF16 ? 8 : 4;                 // V elements per 16-byte vector
  constexpr int EK = MODE == kI8K ? 16 : E;       // K elements per 16-byte vector
  const int cpr = D / EK;  // K vectors per row
  const int si = blockIdx.y;
  const int b = aa.b[si], start = aa.start[si], R = aa.rows[si], row0 = aa.row0[si];
  const int rr0 = aa.rope_row0[si];
  int v_group0, v_groups_per_slab;
  v_groups(BF16, start, R, v_group0, v_groups_per_slab);
  const long long n_k_vecs = (long long)R * Hkv * cpr;
  const long long n_v_vecs = (long long)Hkv * v_groups_per_slab * D;
  const long long n_q_vecs = QB ? (long long)R * Hq * (D / 8) : 0;
  long long tid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  const long long stride = (long long)gridDim.x * blockDim.x;
  long long first = tid;
  if constexpr (MODE == kI8K) {
    // K rows one per wave, then the V vectors
    const int lane = threadIdx.x & (kWave - 1);
    const long long wv = tid / kWave, nw = stride / kWave;
    for (long long rt = wv; rt < (long long)R * Hkv; rt += nw) {
      const int g = (int)(rt % Hkv), row = (int)(rt / Hkv);
      const int j = start + row;
      const float* rowp = k_new + (((size_t)row0 + row) * Hkv + g) * D;
      const float* cr = ROPE ? rope_cos + ((size_t)rr0 + row) * (D >> 1) : nullptr;
      const float* sr = ROPE ? rope_sin + ((size_t)rr0 + row) * (D >> 1) : nullptr;
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;  // bytes
      quantise_row_wave<ROPE>(rowp, cr, sr, D, lane, reinterpret_cast<int8_t*>(k_cache) + slab,
                              k_vec_index(j, 0, D, 16), k_scales + ((size_t)b * Hkv + g) * C + j);
    }
    first = tid + n_k_vecs;  // the vector loop below does V only
  }
  for (long long i = first; i < n_k_vecs + n_v_vecs + n_q_vecs; i += stride) {
    if (QB && i >= n_k_vecs + n_v_vecs) {
      // Q vector: (row, head, c) with c innermost
      const long long iq = i - n_k_vecs - n_v_vecs;
      const int c = (int)(iq % (D / 8));
      const long long t = iq / (D / 8);
      const size_t qrow = ((size_t)row0 + t / Hq) * Hq + (size_t)(t % Hq);
      const float4 a = *reinterpret_cast<const float4*>(q + qrow * D + 8 * c);
      const float4 b = *reinterpret_cast<const float4*>(q + qrow * D + 8 * c + 4);
      float f[8];
      f[0] = a.x * sl2e; f[1] = a.y * sl2e; f[2] = a.z * sl2e; f[3] = a.w * sl2e;
      f[4] = b.x * sl2e; f[5] = b.y * sl2e; f[6] = b.z * sl2e; f[7] = b.w * sl2e;
      qb[qrow * (D / 8) + c] = __builtin_bit_cast(uint4, to_bf16x8(f));
    } else if (i < n_k_vecs) {
      // K vector: (row, g, c) with c innermost
      const int c = (int)(i % cpr);
      long long t = i / cpr;
      const int g = (int)(t % Hkv);
      const int row = (int)(t / Hkv);
      const int j = start + row;
      const float* rowp = k_new + (((size_t)row0 + row) * Hkv + g) * D;
      const float* src = rowp + c * EK;
      const size_t slab = ((size_t)b * Hkv + g) * (size_t)C * D;  // elements
      const size_t vi = k_vec_index(j, c, D, EK);
      float f[E];
      if constexpr (ROPE) {
        // this vector's E dims and their partners in the other half
        const int h = D >> 1;
        const int d0 = c * E, j0 = d0 < h ? d0 : d0 - h;
        const float* cr = rope_cos + ((size_t)rr0 + row) * h + j0;
        const float* sr = rope_sin + ((size_t)rr0 + row) * h + j0;
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 a = *reinterpret_cast<const float4*>(rowp + j0 + e);
          const float4 b = *reinterpret_cast<const float4*>(rowp + j0 + h + e);
          float4 lo, hi;
          rope4(a, b, *reinterpret_cast<const float4*>(cr + e),
                *reinterpret_cast<const float4*>(sr + e), lo, hi);
          const float4 o = d0 < h ? lo : hi;
          f[e] = o.x; f[e + 1] = o.y; f[e + 2] = o.z; f[e + 3] = o.w;
        }
      } else {
#pragma unroll
        for (int e = 0; e < E; e += 4) {
          const float4 a = *reinterpret_cast<const float4*>(src + e);
          f[e] = a.x; f[e + 1] = a.y; f[e + 2] = a.z; f[e + 3] = a.w;
        }
      }
      if constexpr (BF16) {
        uint4 o;
        o.x = pack_bf16x2(f[0], f[1]);
        o.y = pack_bf16x2(f[2], f[3]);
        o.z = pack_bf16x2(f[4], f[5]);
        o.w = pack_bf16x2(f[6], f[7]);
        reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(k_cache) + slab)[vi] = o;
      } else {
        reinterpret_cast<float4*>(reinterpret_cast<float*>(k_cache) + slab)[vi] =
            make_float4(f[0], f[1], f[2], f[3]);
      }
    } else {
      // V vector: (g, group, d) with d innermost; a group spans E positions
      const long long iv = i - n_k_vecs;
      const int d = (int)(iv % D);
      const long long t = iv / D;
      const int gi = (int)(t % v_groups_per_slab) + v_group0;
      const int g = (int)(t / v_groups_per_slab);
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
        vals[s] = have[s] ? v_new[(((size_t)row0 + row) * Hkv + g) * D + d] : 0.f;
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

// Launches the append for the sessions of tables L (grid: blocks x
// sessions of a table).
static hipError_t launch_append_tables(const Shape& s, void* k_cache, void* v_cache,
                                       const float* k_new, const float* v_new,
                                       const float* rope_cos, const float* rope_sin,
                                       const std::vector<AppendArg>& L, hipStream_t stream,
                                       const float* q = nullptr, void* qb = nullptr,
                                       float sl2e = 0.f) {
  const int mode = s.kv_dtype;
  const bool bf16 = mode != kF32;                      // V layout
  const int E = mode == kF32 ? 4 : mode == kBF16 ? 8 : 16;   // K elements per vector
  const bool rope = rope_cos != nullptr;
  float* k_scales = k_scale_array(s, k_cache);
  for (const AppendArg& aa : L) {
    long long most = 0;  // vectors of the largest session
    for (int i = 0; i < aa.n; ++i) {
      int g0, ng;
      v_groups(bf16, aa.start[i], aa.rows[i], g0, ng);
      // threads: one per K vector (int8 K: one wave per row) and per V vector
      const long long nk = mode == kI8K ? (long long)aa.rows[i] * s.num_kv_heads * kWave
                                        : (long long)aa.rows[i] * s.num_kv_heads * (s.head_dim / E);
      const long long nq = qb ? (long long)aa.rows[i] * s.num_q_heads * (s.head_dim / 8) : 0;
      const long long n = nk + (long long)s.num_kv_heads * ng * s.head_dim + nq;
      if (n > most) most = n;
    }
    long long blocks = (most + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    const dim3 grid((unsigned)blocks, aa.n);
    auto go = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, k_cache, v_cache, k_new, v_new,
                         rope_cos, rope_sin, k_scales, s.num_kv_heads, s.head_dim, s.capacity, aa,
                         q, static_cast<uint4*>(qb), s.num_q_heads, sl2e);
    };
    if (qb) {
      if (mode != kBF16 || rope) return hipErrorInvalidValue;
      go(append_kernel<kBF16, false, true>);
    } else if (mode == kI8K) rope ? go(append_kernel<kI8K, true>) : go(append_kernel<kI8K, false>);
    else if (mode == kBF16) rope ? go(append_kernel<kBF16, true>) : go(append_kernel<kBF16, false>);
    else rope ? go(append_kernel<kF32, true>) : go(append_kernel<kF32, false>);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Sessions with rows, kAppendSessions per table, packed rows in session
// order; cos / sin rows shared by all sessions (shared_rope) or packed like
// the rows.
template <class Rows, class Start>
static std::vector<AppendArg> append_tables(int batch, Rows rows_of, Start start_of,
                                            bool shared_rope) {
  std::vector<AppendArg> L;
  AppendArg cur{};
  long long row = 0;
  for (int b = 0; b < batch; ++b) {
    const int R = rows_of(b);
    if (R <= 0) continue;
    if (cur.n == kAppendSessions) {
      L.push_back(cur);
      cur = AppendArg{};
    }
    const int i = cur.n++;
    cur.b[i] = b;
    cur.start[i] = start_of(b);
    cur.rows[i] = R;
    cur.row0[i] = (int)row;
    cur.rope_row0[i] = shared_rope ? 0 : (int)row;
    row += R;
  }
  if (cur.n > 0) L.push_back(cur);
  return L;
}

hipError_t launch_append(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                         const float* v_new, int start, int R, hipStream_t stream,
                         const float* rope_cos, const float* rope_sin) {
  const auto L = append_tables(
      s.batch, [&](int) { return R; }, [&](int) { return start; }, true);
  return launch_append_tables(s, k_cache, v_cache, k_new, v_new, rope_cos, rope_sin, L, stream);
}

hipError_t launch_append_q(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                           const float* v_new, int start, int R, const float* q, void* qb,
                           float scale, hipStream_t stream) {
  const auto L = append_tables(
      s.batch, [&](int) { return R; }, [&](int) { return start; }, true);
  return launch_append_tables(s, k_cache, v_cache, k_new, v_new, nullptr, nullptr, L, stream, q,
                              qb, scale * kLog2e);
}

hipError_t launch_append_ragged(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                                const float* v_new, const int32_t* start, const int32_t* rows,
                                hipStream_t stream, const float* rope_cos,
                                const float* rope_sin) {
  const auto L = append_tables(
      s.batch, [&](int b) { return rows[b]; }, [&](int b) { return start[b]; }, false);
  return launch_append_tables(s, k_cache, v_cache, k_new, v_new, rope_cos, rope_sin, L, stream);
}

// Rotary embedding of query rows: x, y f32 [B][R][H][D] (y may be x), each
// element rotated by its row's cos / sin ([R][D/2]) exactly as the append's
// K rows are.  One thread per 4 output elements; all of a pair's inputs are
// read before either output is written, so in-place use is safe.
__global__ __launch_bounds__(256) void rope_rows_kernel(const float* __restrict__ x, float* y,
                                                        const float* __restrict__ rope_cos,
                                                        const float* __restrict__ rope_sin,
                                                        long long n_pairs4, int R, int H, int D) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n_pairs4) return;
  // pair group i: 4 consecutive dims j .. j+3 of the first half of one
  // (b, r, head) row, with their partners j + D/2 ..
  const int h2 = D >> 1;
  const int q4 = h2 >> 2;
  const int j = (int)(i % q4) * 4;
  const long long rowi = i / q4;  // (b, r, head) row index
  const int r = (int)((rowi / H) % R);
  const float* xr = x + rowi * D;
  float* yr = y + rowi * D;
  const float* cr = rope_cos + (size_t)r * h2;
  const float* sr = rope_sin + (size_t)r * h2;
  float4 lo, hi;
  rope4(*reinterpret_cast<const float4*>(xr + j), *reinterpret_cast<const float4*>(xr + j + h2),
        *reinterpret_cast<const float4*>(cr + j), *reinterpret_cast<const float4*>(sr + j), lo, hi);
  *reinterpret_cast<float4*>(yr + j) = lo;
  *reinterpret_cast<float4*>(yr + j + h2) = hi;
}

hipError_t launch_rope_rows(const float* x, float* y, const float* rope_cos,
                            const float* rope_sin, int B, int R, int H, int D,
                            hipStream_t stream) {
  const long long n = (long long)B * R * H * (D / 8);
  const int threads = 256;
  const long long blocks = (n + threads - 1) / threads;
  hipLaunchKernelGGL(rope_rows_kernel, dim3((unsigned)blocks), dim3(threads), 0, stream, x, y,
                     rope_cos, rope_sin, n, R, H, D);
  return hipGetLastError();
}

}  // namespace ka
