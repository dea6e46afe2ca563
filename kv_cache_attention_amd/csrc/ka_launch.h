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

hipError_t launch_append(const Shape& s, void* k_cache, void* v_cache, const float* k_new,
                         const float* v_new, int start, int R, hipStream_t stream);

// ---- prefill
struct PrefillPlan {
  int m_tiles;   // ceil(R * G / 128)
  int splits;    // key-range splits per m-tile (1 = no workspace)
  size_t workspace_bytes;
};
PrefillPlan plan_prefill(const Shape& s, int start, int R);
size_t prefill_workspace_bound(const Shape& s, int max_rows);
hipError_t launch_prefill(const Shape& s, const PrefillPlan& p, const float* q,
                          const void* k_cache, const void* v_cache, float* out, int start, int R,
                          float scale, void* workspace, hipStream_t stream);

// ---- decode
struct DecodePlan {
  int heads_per_wg;  // query heads one workgroup serves (divides G)
  int head_groups;   // G / heads_per_wg
  int splits;        // context splits per (session, KV head, head group)
  size_t workspace_bytes;
};
DecodePlan plan_decode(const Shape& s, int max_ctx);
hipError_t launch_decode(const Shape& s, const DecodePlan& p, const float* q,
                         const void* k_cache, const void* v_cache, float* out,
                         const int32_t* ctx_host, float scale, void* workspace,
                         hipStream_t stream);

}  // namespace ka
