// Internal launchers of the attention kernels.  Arguments are validated by
// the C-ABI layer (api.hip) before any of these is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace ka {

struct Shape {
  int batch, num_q_heads, num_kv_heads, head_dim, capacity, kv_dtype;
};

// Most sessions one decode launch carries (their context lengths travel as a
// kernel argument); larger batches are issued as several launches.
constexpr int kMaxDecodeBatchPerLaunch = 256;

struct CtxArg {
  int32_t ctx[kMaxDecodeBatchPerLaunch];
};

// int8-K caches: the row scales follow the codes of every slab in the K
// buffer, [B][Hkv][C] f32 from byte B * Hkv * C * D (null for other dtypes).
inline float* k_scale_array(const Shape& s, const void* k_cache) {
  if (s.kv_dtype != 2) return nullptr;
  return reinterpret_cast<float*>(const_cast<unsigned char*>(static_cast<const unsigned char*>(k_cache)) +
                                  (size_t)s.batch * s.num_kv_heads * s.capacity * s.head_dim);
}

// rope_cos / rope_sin: null for a plain append, else [R][D/2] rows that rotate
// each new K row before it is stored.
hipError_t launch_append(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                         const float* v_new, int start, int R, hipStream_t stream,
                         const float* rope_cos = nullptr, const float* rope_sin = nullptr);
// The append of a uniform chunk on a bf16 cache that also writes the chunk's
// Q rows (f32 [B][R][Hq][D]) to qb as bf16 of q * scale * log2 e, rounded as
// the prefill kernel rounds its Q operands (for launch_prefill's qb).
hipError_t launch_append_q(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                           const float* v_new, int start, int R, const float* q, void* qb,
                           float scale, hipStream_t stream);
// Ragged: session b appends rows[b] rows (0: none) at positions start[b] ..,
// rows packed in session order in k_new / v_new ([sum rows][Hkv][D]) and in
// rope_cos / rope_sin when given.  start / rows are host arrays [B].
hipError_t launch_append_ragged(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                                const float* v_new, const int32_t* start, const int32_t* rows,
                                hipStream_t stream, const float* rope_cos = nullptr,
                                const float* rope_sin = nullptr);
// Rotary embedding of f32 rows x -> y ([B][R][H][D], y may be x).
hipError_t launch_rope_rows(const float* x, float* y, const float* rope_cos,
                            const float* rope_sin, int B, int R, int H, int D,
                            hipStream_t stream);

// Split-context plan of the decode kernels.  On the bf16 MFMA kernel a
// workgroup's columns are heads_per_wg (row, head) pairs -- one row: heads.
struct DecodePlan {
  int heads_per_wg;  // columns one workgroup serves
  int head_groups;   // workgroups sharing a KV head's columns
  int splits;        // context splits per (session, KV head, head group)
  size_t workspace_bytes;
};

// ---- prefill
struct PrefillPlan {
  int m_tiles;   // ceil(R * G / 128); 0: a few-row chunk served by the decode kernel
  int splits;    // key-range splits per m-tile (1 = no workspace)
  size_t workspace_bytes;
  DecodePlan rows;  // the decode kernel's plan when m_tiles == 0
};
PrefillPlan plan_prefill(const Shape& s, int start, int R);
size_t prefill_workspace_bound(const Shape& s, int max_rows);
// qb (bf16 caches, M-tile plans only; null otherwise): Q already scaled and
// rounded by launch_append_q, [B][R][Hq][D] bf16, read instead of q.
hipError_t launch_prefill(const Shape& s, const PrefillPlan& p, const float* q,
                          const void* k_cache, const void* v_cache, float* out, int start, int R,
                          float scale, void* workspace, hipStream_t stream,
                          const void* qb = nullptr);
// Ragged prefill: session b's rows[b] rows (0: none) at positions start[b] ..,
// packed in session order in q / out ([sum rows][Hq][D]); all sessions' tiles
// share each launch.  start / rows are host arrays [B].
size_t prefill_ragged_workspace(const Shape& s, const int32_t* start, const int32_t* rows);
size_t prefill_ragged_workspace_bound(const Shape& s, long long max_total_rows);
hipError_t launch_prefill_ragged(const Shape& s, const float* q, const void* k_cache,
                                 const void* v_cache, float* out, const int32_t* start,
                                 const int32_t* rows, float scale, void* workspace,
                                 hipStream_t stream);

// ---- decode
DecodePlan plan_decode(const Shape& s, int max_ctx);
// k_new / v_new (optional, [B][Hkv][D] f32): the decode step's new rows, at
// position ctx - 1 of each session; the attention kernel stores them as the
// append would and attends to them (no separate append launch).
hipError_t launch_decode(const Shape& s, const DecodePlan& p, const float* q, void* k_cache,
                         void* v_cache, float* out, const int32_t* ctx_host, float scale,
                         void* workspace, hipStream_t stream, const float* k_new = nullptr,
                         const float* v_new = nullptr);

// ---- chunks of a few rows on bf16 caches: the decode kernel, its 16 MFMA
// columns taken by (row, head) pairs of a KV group (row p / G, head p % G),
// each pair with its own causal limit; R rows at positions start .. start + R - 1.
DecodePlan plan_rows(const Shape& s, int R, int ctx);
hipError_t launch_rows(const Shape& s, const DecodePlan& p, const float* q, const void* k_cache,
                       const void* v_cache, float* out, int start, int R, float scale,
                       void* workspace, hipStream_t stream);

// ---- int8 scores: the device self-test (run once per device, then cached).
// *passed tells whether the int8 MFMA and its emulation both gave the known
// answer; *why is a static description of the outcome.
hipError_t int8_self_test(bool* passed, const char** why);

}  // namespace ka
