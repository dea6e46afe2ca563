// C ABI of the attention library: argument validation (always before any
// work is enqueued, so a rejected call changes nothing), plan selection and
// the per-thread error text.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <vector>

#include "ka_attn.h"
#include "ka_launch.h"

namespace {

thread_local char g_last_error[512] = "";

ka_status fail(ka_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return st;
}

ka_status ok() {
  g_last_error[0] = '\0';
  return KA_OK;
}

ka_status hip_fail(hipError_t e, const char* where) {
  return fail(KA_ERR_HIP, "%s: %s (%s)", where, hipGetErrorName(e), hipGetErrorString(e));
}

// Checks a shape; on success fills *out.
ka_status check_shape(const ka_attn_shape* s, ka::Shape* out) {
  if (!s) return fail(KA_ERR_INVALID_ARGUMENT, "shape is NULL");
  if (s->batch < 1) return fail(KA_ERR_INVALID_ARGUMENT, "batch must be >= 1 (got %d)", s->batch);
  if (s->num_q_heads < 1 || s->num_kv_heads < 1)
    return fail(KA_ERR_INVALID_ARGUMENT, "head counts must be >= 1 (got Hq=%d, Hkv=%d)",
                s->num_q_heads, s->num_kv_heads);
  if (s->num_q_heads % s->num_kv_heads != 0)
    return fail(KA_ERR_INVALID_ARGUMENT, "num_q_heads %d is not a multiple of num_kv_heads %d",
                s->num_q_heads, s->num_kv_heads);
  if (s->head_dim != 64 && s->head_dim != 128 && s->head_dim != 256)
    return fail(KA_ERR_UNSUPPORTED, "head_dim %d not supported (64, 128 or 256)", s->head_dim);
  if (s->kv_dtype != KA_DTYPE_F32 && s->kv_dtype != KA_DTYPE_BF16 && s->kv_dtype != KA_DTYPE_I8K)
    return fail(KA_ERR_UNSUPPORTED, "kv_dtype %d not supported (0 = f32, 1 = bf16, 2 = int8 K)",
                s->kv_dtype);
  if (s->num_q_heads > KA_ATTN_MAX_Q_HEADS)
    return fail(KA_ERR_OUT_OF_RANGE, "num_q_heads %d exceeds %d", s->num_q_heads,
                KA_ATTN_MAX_Q_HEADS);
  if (s->batch > KA_ATTN_MAX_BATCH)
    return fail(KA_ERR_OUT_OF_RANGE, "batch %d exceeds %d", s->batch, KA_ATTN_MAX_BATCH);
  if (s->capacity > KA_ATTN_MAX_CAPACITY)
    return fail(KA_ERR_OUT_OF_RANGE, "capacity %d exceeds %d", s->capacity, KA_ATTN_MAX_CAPACITY);
  if (s->capacity < 64 || s->capacity % 64 != 0)
    return fail(KA_ERR_INVALID_ARGUMENT, "capacity %d must be a positive multiple of 64",
                s->capacity);
  *out = ka::Shape{s->batch, s->num_q_heads, s->num_kv_heads, s->head_dim, s->capacity,
                   s->kv_dtype};
  return KA_OK;
}

ka_status check_scale(float scale) {
  if (!std::isfinite(scale) || !(scale > 0.f))
    return fail(KA_ERR_INVALID_ARGUMENT, "scale must be finite and > 0 (got %g)", (double)scale);
  return KA_OK;
}

// Per-session chunks of a ragged call: host arrays start / rows of B entries,
// rows >= 0, start >= 0, start + rows <= capacity.  *total gets the row sum.
ka_status check_ragged(const ka::Shape& sh, const int32_t* start, const int32_t* rows,
                       long long* total) {
  if (!start || !rows) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos / row_count is NULL");
  long long t = 0;
  for (int b = 0; b < sh.batch; ++b) {
    if (rows[b] < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count[%d] = %d < 0", b, rows[b]);
    if (start[b] < 0) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos[%d] = %d < 0", b, start[b]);
    if ((long long)start[b] + rows[b] > sh.capacity)
      return fail(KA_ERR_OUT_OF_RANGE, "start_pos[%d] %d + row_count[%d] %d exceeds capacity %d", b,
                  start[b], b, rows[b], sh.capacity);
    t += rows[b];
  }
  if (t > 0x7fffffffLL) return fail(KA_ERR_OUT_OF_RANGE, "%lld rows in all exceed 2^31 - 1", t);
  *total = t;
  return KA_OK;
}

// One buffer: f32 4 bytes per element, bf16 2; int8-K caches size both
// buffers as the bf16 V buffer, which also holds the K codes (1 byte per
// element) and their row scales (4 bytes per row).
size_t cache_bytes(const ka::Shape& s) {
  return (size_t)s.batch * s.num_kv_heads * (size_t)s.capacity * s.head_dim *
         (s.kv_dtype == KA_DTYPE_F32 ? 4 : 2);
}

// Calls that compute int8 scores first make sure the device passed the
// self-test (run at the first such call on each device).
ka_status check_int8(const ka::Shape& sh) {
  if (sh.kv_dtype != KA_DTYPE_I8K) return KA_OK;
  bool passed = false;
  const char* why = "";
  const hipError_t e = ka::int8_self_test(&passed, &why);
  if (e != hipSuccess) return hip_fail(e, "int8 self-test");
  if (!passed) return fail(KA_ERR_UNSUPPORTED, "%s", why);
  return KA_OK;
}

// Scratch of the allocation-free decode step: the split partials live in this
// file-scope device array instead of a caller's workspace.  Each device that
// runs the library holds its own copy until the process ends; in host code
// the name stands for no device address, so its address on a device is taken
// once (hipGetSymbolAddress, with that device current) and kept per device.
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ka_status scratch_of_current_device(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(KA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return KA_OK;
}

}  // namespace

extern "C" {

int32_t ka_attn_abi_version(void) { return KA_ATTN_ABI_VERSION; }

size_t ka_attn_cache_bytes(const ka_attn_shape* s) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  return cache_bytes(sh);
}

ka_status ka_attn_append_kv(const ka_attn_shape* s, void* k_cache, void* v_cache,
                            const float* k_new, const float* v_new, int32_t start_pos,
                            int32_t row_count, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (row_count < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count %d < 0", row_count);
  if (start_pos < 0) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos %d < 0", start_pos);
  if ((long long)start_pos + row_count > sh.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "start_pos %d + row_count %d exceeds capacity %d",
                start_pos, row_count, sh.capacity);
  if (row_count == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  hipError_t e = ka::launch_append(sh, k_cache, v_cache, k_new, v_new, start_pos, row_count,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

ka_status ka_attn_append_kv_rope(const ka_attn_shape* s, void* k_cache, void* v_cache,
                                 const float* k_new, const float* v_new, const float* rope_cos,
                                 const float* rope_sin, int32_t start_pos, int32_t row_count,
                                 void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (row_count < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count %d < 0", row_count);
  if (start_pos < 0) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos %d < 0", start_pos);
  if ((long long)start_pos + row_count > sh.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "start_pos %d + row_count %d exceeds capacity %d",
                start_pos, row_count, sh.capacity);
  if (row_count == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !rope_cos || !rope_sin)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  hipError_t e = ka::launch_append(sh, k_cache, v_cache, k_new, v_new, start_pos, row_count,
                                   reinterpret_cast<hipStream_t>(stream), rope_cos, rope_sin);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

ka_status ka_attn_append_kv_ragged(const ka_attn_shape* s, void* k_cache, void* v_cache,
                                   const float* k_new, const float* v_new, const float* rope_cos,
                                   const float* rope_sin, const int32_t* start_pos,
                                   const int32_t* row_count, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  long long total = 0;
  if ((st = check_ragged(sh, start_pos, row_count, &total)) != KA_OK) return st;
  if ((rope_cos == nullptr) != (rope_sin == nullptr))
    return fail(KA_ERR_INVALID_ARGUMENT, "rope_cos and rope_sin must both be given or both NULL");
  if (total == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  hipError_t e = ka::launch_append_ragged(sh, k_cache, v_cache, k_new, v_new, start_pos, row_count,
                                          reinterpret_cast<hipStream_t>(stream), rope_cos, rope_sin);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  return ok();
}

ka_status ka_attn_rope_rows(const ka_attn_shape* s, const float* x, float* y,
                            const float* rope_cos, const float* rope_sin, int32_t row_count,
                            void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (row_count < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count %d < 0", row_count);
  if (row_count == 0) return ok();
  if (!x || !y || !rope_cos || !rope_sin) return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  hipError_t e = ka::launch_rope_rows(x, y, rope_cos, rope_sin, sh.batch, row_count,
                                      sh.num_q_heads, sh.head_dim,
                                      reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rope launch");
  return ok();
}

size_t ka_attn_prefill_workspace_bytes(const ka_attn_shape* s, int32_t max_rows) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  return ka::prefill_workspace_bound(sh, max_rows);
}

size_t ka_attn_prefill_workspace_need(const ka_attn_shape* s, int32_t start_pos,
                                      int32_t row_count) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  if (start_pos < 0 || row_count <= 0 || (long long)start_pos + row_count > sh.capacity) return 0;
  return ka::plan_prefill(sh, start_pos, row_count).workspace_bytes;
}

ka_status ka_attn_prefill_chunk(const ka_attn_shape* s, const float* q, const void* k_cache,
                                const void* v_cache, float* out, int32_t start_pos,
                                int32_t row_count, float scale, void* workspace,
                                size_t workspace_bytes, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (row_count < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count %d < 0", row_count);
  if (start_pos < 0) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos %d < 0", start_pos);
  if ((long long)start_pos + row_count > sh.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "start_pos %d + row_count %d exceeds capacity %d",
                start_pos, row_count, sh.capacity);
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (row_count == 0) return ok();
  if (!q || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const ka::PrefillPlan plan = ka::plan_prefill(sh, start_pos, row_count);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(KA_ERR_WORKSPACE, "prefill needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_int8(sh)) != KA_OK) return st;
  hipError_t e = ka::launch_prefill(sh, plan, q, k_cache, v_cache, out, start_pos, row_count,
                                    scale, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

}  // extern "C"

namespace {

// The fused append and prefill: on bf16 caches with an M-tile plan the append
// also writes the chunk's Q, scaled and rounded, for the prefill kernel to
// read (half the bytes of f32 Q, and no conversion in the prefill); it sits in
// the workspace behind the split partials, from a 256-byte boundary.
size_t round_up_256(size_t n) { return (n + 255) & ~(size_t)255; }
bool fused_uses_qb(const ka::Shape& sh, const ka::PrefillPlan& plan) {
  return sh.kv_dtype == KA_DTYPE_BF16 && plan.m_tiles > 0;
}
size_t qb_bytes(const ka::Shape& sh, long long rows) {
  return (size_t)sh.batch * (size_t)rows * sh.num_q_heads * sh.head_dim * 2;
}
size_t fused_need(const ka::Shape& sh, const ka::PrefillPlan& plan, int rows) {
  if (!fused_uses_qb(sh, plan)) return plan.workspace_bytes;
  return round_up_256(plan.workspace_bytes) + qb_bytes(sh, rows);
}

}  // namespace

extern "C" {

size_t ka_attn_append_prefill_workspace_bytes(const ka_attn_shape* s, int32_t max_rows) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK || max_rows <= 0) return 0;
  const int rows = max_rows < sh.capacity ? max_rows : sh.capacity;
  const size_t part = ka::prefill_workspace_bound(sh, rows);
  if (sh.kv_dtype != KA_DTYPE_BF16) return part;
  return round_up_256(part) + qb_bytes(sh, rows);
}

size_t ka_attn_append_prefill_workspace_need(const ka_attn_shape* s, int32_t start_pos,
                                             int32_t row_count) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  if (start_pos < 0 || row_count <= 0 || (long long)start_pos + row_count > sh.capacity) return 0;
  return fused_need(sh, ka::plan_prefill(sh, start_pos, row_count), row_count);
}

ka_status ka_attn_append_prefill_chunk(const ka_attn_shape* s, const float* q, const float* k_new,
                                       const float* v_new, void* k_cache, void* v_cache,
                                       float* out, int32_t start_pos, int32_t row_count,
                                       float scale, void* workspace, size_t workspace_bytes,
                                       void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (row_count < 0) return fail(KA_ERR_INVALID_ARGUMENT, "row_count %d < 0", row_count);
  if (start_pos < 0) return fail(KA_ERR_INVALID_ARGUMENT, "start_pos %d < 0", start_pos);
  if ((long long)start_pos + row_count > sh.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "start_pos %d + row_count %d exceeds capacity %d",
                start_pos, row_count, sh.capacity);
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (row_count == 0) return ok();
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const ka::PrefillPlan plan = ka::plan_prefill(sh, start_pos, row_count);
  const size_t need = fused_need(sh, plan, row_count);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KA_ERR_WORKSPACE, "append and prefill need %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_int8(sh)) != KA_OK) return st;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  void* qb = nullptr;
  hipError_t e;
  if (fused_uses_qb(sh, plan)) {
    qb = static_cast<unsigned char*>(workspace) + round_up_256(plan.workspace_bytes);
    e = ka::launch_append_q(sh, k_cache, v_cache, k_new, v_new, start_pos, row_count, q, qb, scale,
                            hs);
  } else {
    e = ka::launch_append(sh, k_cache, v_cache, k_new, v_new, start_pos, row_count, hs);
  }
  if (e != hipSuccess) return hip_fail(e, "append launch");
  e = ka::launch_prefill(sh, plan, q, k_cache, v_cache, out, start_pos, row_count, scale,
                         workspace, hs, qb);
  if (e != hipSuccess) return hip_fail(e, "prefill launch");
  return ok();
}

size_t ka_attn_prefill_ragged_workspace_bytes(const ka_attn_shape* s, int64_t max_total_rows) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  return ka::prefill_ragged_workspace_bound(sh, max_total_rows);
}

size_t ka_attn_prefill_ragged_workspace_need(const ka_attn_shape* s, const int32_t* start_pos,
                                             const int32_t* row_count) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  long long total = 0;
  if (check_ragged(sh, start_pos, row_count, &total) != KA_OK || total == 0) return 0;
  return ka::prefill_ragged_workspace(sh, start_pos, row_count);
}

ka_status ka_attn_prefill_ragged(const ka_attn_shape* s, const float* q, const void* k_cache,
                                 const void* v_cache, float* out, const int32_t* start_pos,
                                 const int32_t* row_count, float scale, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  long long total = 0;
  if ((st = check_ragged(sh, start_pos, row_count, &total)) != KA_OK) return st;
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (total == 0) return ok();
  if (!q || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const size_t need = ka::prefill_ragged_workspace(sh, start_pos, row_count);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(KA_ERR_WORKSPACE, "ragged prefill needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_int8(sh)) != KA_OK) return st;
  hipError_t e = ka::launch_prefill_ragged(sh, q, k_cache, v_cache, out, start_pos, row_count,
                                           scale, workspace, reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "ragged prefill launch");
  return ok();
}

ka_status ka_attn_session_memory(const ka_attn_shape* s, int32_t max_chunk_rows,
                                 ka_attn_memory* m) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (!m) return fail(KA_ERR_INVALID_ARGUMENT, "memory estimate pointer is NULL");
  if (max_chunk_rows < 1 || max_chunk_rows > sh.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "max_chunk_rows %d outside 1..capacity (%d)", max_chunk_rows,
                sh.capacity);
  m->cache_bytes = 2 * cache_bytes(sh);
  m->prefill_workspace_bytes = ka::prefill_workspace_bound(sh, max_chunk_rows);
  m->decode_workspace_bytes = ka::plan_decode(sh, sh.capacity).workspace_bytes;
  m->chunk_io_bytes = (size_t)sh.batch * max_chunk_rows *
                      (2 * (size_t)sh.num_q_heads + 2 * (size_t)sh.num_kv_heads) * sh.head_dim *
                      sizeof(float);
  const size_t ws = m->prefill_workspace_bytes > m->decode_workspace_bytes
                        ? m->prefill_workspace_bytes
                        : m->decode_workspace_bytes;
  m->total_bytes = m->cache_bytes + ws + m->chunk_io_bytes;
  return ok();
}

ka_status ka_attn_cache_resize(const ka_attn_shape* src, const void* src_k, const void* src_v,
                               const ka_attn_shape* dst, void* dst_k, void* dst_v, int32_t rows,
                               void* stream) {
  ka::Shape a, b;
  ka_status st = check_shape(src, &a);
  if (st != KA_OK) return st;
  if ((st = check_shape(dst, &b)) != KA_OK) return st;
  if (a.batch != b.batch || a.num_q_heads != b.num_q_heads || a.num_kv_heads != b.num_kv_heads ||
      a.head_dim != b.head_dim || a.kv_dtype != b.kv_dtype)
    return fail(KA_ERR_INVALID_ARGUMENT, "source and destination differ in more than capacity");
  if (rows < 0) return fail(KA_ERR_INVALID_ARGUMENT, "rows %d < 0", rows);
  if (rows > a.capacity || rows > b.capacity)
    return fail(KA_ERR_OUT_OF_RANGE, "rows %d exceed a capacity (%d -> %d)", rows, a.capacity,
                b.capacity);
  if (rows == 0) return ok();
  if (!src_k || !src_v || !dst_k || !dst_v)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  const size_t es = a.kv_dtype == KA_DTYPE_F32 ? 4 : 2;               // V (and f32 / bf16 K)
  const size_t ek = a.kv_dtype == KA_DTYPE_I8K ? 1 : es;               // K codes
  const size_t src_slab = (size_t)a.capacity * a.head_dim * es;
  const size_t dst_slab = (size_t)b.capacity * b.head_dim * es;
  const size_t nslab = (size_t)a.batch * a.num_kv_heads;
  // the two caches must not overlap (a copy in place is not a resize)
  auto apart = [&](const void* x, const void* y, size_t nx, size_t ny) {
    const char* p = static_cast<const char*>(x);
    const char* q = static_cast<const char*>(y);
    return p + nx <= q || q + ny <= p;
  };
  if (!apart(src_k, dst_k, nslab * src_slab, nslab * dst_slab) ||
      !apart(src_v, dst_v, nslab * src_slab, nslab * dst_slab) ||
      !apart(src_k, dst_v, nslab * src_slab, nslab * dst_slab) ||
      !apart(src_v, dst_k, nslab * src_slab, nslab * dst_slab))
    return fail(KA_ERR_INVALID_ARGUMENT, "source and destination caches overlap");
  // positions 0 .. rows - 1 of a slab are a prefix of it in both layouts:
  // whole 64-position K blocks, whole V groups (32 positions for bf16, 4 for
  // f32); both capacities are multiples of 64 >= rows, so the rounded
  // prefix fits either slab
  const size_t k_pos = ((size_t)rows + 63) / 64 * 64;
  const size_t v_unit = a.kv_dtype == KA_DTYPE_F32 ? 4 : 32;  // V in the bf16 layout unless f32
  const size_t v_pos = ((size_t)rows + v_unit - 1) / v_unit * v_unit;
  const hipStream_t hs = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpy2DAsync(dst_k, (size_t)b.capacity * b.head_dim * ek, src_k,
                                  (size_t)a.capacity * a.head_dim * ek, k_pos * a.head_dim * ek,
                                  nslab, hipMemcpyDeviceToDevice, hs);
  if (e == hipSuccess && a.kv_dtype == KA_DTYPE_I8K)  // the row scales: [B][Hkv][C] f32
    e = hipMemcpy2DAsync(ka::k_scale_array(b, dst_k), (size_t)b.capacity * 4,
                         ka::k_scale_array(a, src_k), (size_t)a.capacity * 4, (size_t)rows * 4,
                         nslab, hipMemcpyDeviceToDevice, hs);
  if (e == hipSuccess)
    e = hipMemcpy2DAsync(dst_v, dst_slab, src_v, src_slab, v_pos * a.head_dim * es, nslab,
                         hipMemcpyDeviceToDevice, hs);
  if (e != hipSuccess) return hip_fail(e, "cache resize copy");
  return ok();
}

ka_status ka_attn_int8_self_test(void) {
  bool passed = false;
  const char* why = "";
  const hipError_t e = ka::int8_self_test(&passed, &why);
  if (e != hipSuccess) return hip_fail(e, "int8 self-test");
  if (!passed) return fail(KA_ERR_UNSUPPORTED, "%s", why);
  return ok();
}

size_t ka_attn_decode_workspace_bytes(const ka_attn_shape* s, int32_t max_ctx_len) {
  ka::Shape sh;
  if (check_shape(s, &sh) != KA_OK) return 0;
  if (max_ctx_len < 1) return 0;
  if (max_ctx_len > sh.capacity) max_ctx_len = sh.capacity;
  return ka::plan_decode(sh, max_ctx_len).workspace_bytes;
}

ka_status ka_attn_decode(const ka_attn_shape* s, const float* q, const void* k_cache,
                         const void* v_cache, float* out, const int32_t* ctx_len, float scale,
                         void* workspace, size_t workspace_bytes, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (!ctx_len) return fail(KA_ERR_INVALID_ARGUMENT, "ctx_len is NULL");
  int max_ctx = 0;
  for (int b = 0; b < sh.batch; ++b) {
    if (ctx_len[b] < 1 || ctx_len[b] > sh.capacity)
      return fail(KA_ERR_OUT_OF_RANGE, "ctx_len[%d] = %d outside 1..capacity (%d)", b, ctx_len[b],
                  sh.capacity);
    if (ctx_len[b] > max_ctx) max_ctx = ctx_len[b];
  }
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (!q || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const ka::DecodePlan plan = ka::plan_decode(sh, max_ctx);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(KA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_int8(sh)) != KA_OK) return st;
  hipError_t e = ka::launch_decode(sh, plan, q, const_cast<void*>(k_cache),
                                   const_cast<void*>(v_cache), out, ctx_len, scale, workspace,
                                   reinterpret_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return ok();
}

ka_status ka_attn_decode_step(const ka_attn_shape* s, const float* q, const float* k_new,
                              const float* v_new, void* k_cache, void* v_cache, float* out,
                              const int32_t* pos, float scale, void* workspace,
                              size_t workspace_bytes, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (!pos) return fail(KA_ERR_INVALID_ARGUMENT, "pos is NULL");
  std::vector<int32_t> ctx(sh.batch);
  int max_ctx = 0;
  for (int b = 0; b < sh.batch; ++b) {
    if (pos[b] < 0 || pos[b] >= sh.capacity)
      return fail(KA_ERR_OUT_OF_RANGE, "pos[%d] = %d outside 0..capacity-1 (%d)", b, pos[b],
                  sh.capacity - 1);
    ctx[b] = pos[b] + 1;
    if (ctx[b] > max_ctx) max_ctx = ctx[b];
  }
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const ka::DecodePlan plan = ka::plan_decode(sh, max_ctx);
  if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
    return fail(KA_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", plan.workspace_bytes,
                workspace ? workspace_bytes : (size_t)0);
  if ((st = check_int8(sh)) != KA_OK) return st;
  hipError_t e = ka::launch_decode(sh, plan, q, k_cache, v_cache, out, ctx.data(), scale,
                                   workspace, reinterpret_cast<hipStream_t>(stream), k_new, v_new);
  if (e != hipSuccess) return hip_fail(e, "decode step launch");
  return ok();
}

size_t ka_attn_decode_step_noalloc_max_bytes(void) { return kScratchBytes; }

ka_status ka_attn_decode_step_noalloc(const ka_attn_shape* s, const float* q, const float* k_new,
                                      const float* v_new, void* k_cache, void* v_cache,
                                      float* out, const int32_t* pos, float scale, void* stream) {
  ka::Shape sh;
  ka_status st = check_shape(s, &sh);
  if (st != KA_OK) return st;
  if (!pos) return fail(KA_ERR_INVALID_ARGUMENT, "pos is NULL");
  int max_ctx = 0;
  for (int b = 0; b < sh.batch; ++b) {
    if (pos[b] < 0 || pos[b] >= sh.capacity)
      return fail(KA_ERR_OUT_OF_RANGE, "pos[%d] = %d outside 0..capacity-1 (%d)", b, pos[b],
                  sh.capacity - 1);
    if (pos[b] + 1 > max_ctx) max_ctx = pos[b] + 1;
  }
  if ((st = check_scale(scale)) != KA_OK) return st;
  if (!q || !k_new || !v_new || !k_cache || !v_cache || !out)
    return fail(KA_ERR_INVALID_ARGUMENT, "null tensor pointer");
  if ((const void*)q == (const void*)out)
    return fail(KA_ERR_INVALID_ARGUMENT, "out must not alias q");
  const size_t need = ka::plan_decode(sh, max_ctx).workspace_bytes;
  if (need > kScratchBytes)
    return fail(KA_ERR_WORKSPACE,
                "decode step needs %zu scratch bytes, more than the %zu the allocation-free "
                "variant holds; use ka_attn_decode_step with a workspace",
                need, kScratchBytes);
  void* ws = nullptr;
  if (need > 0 && (st = scratch_of_current_device(&ws)) != KA_OK) return st;
  return ka_attn_decode_step(s, q, k_new, v_new, k_cache, v_cache, out, pos, scale, ws, need,
                             stream);
}

const char* ka_attn_status_string(int32_t status) {
  switch (status) {
    case KA_OK: return "KA_OK";
    case KA_ERR_INVALID_ARGUMENT: return "KA_ERR_INVALID_ARGUMENT";
    case KA_ERR_OUT_OF_RANGE: return "KA_ERR_OUT_OF_RANGE";
    case KA_ERR_UNSUPPORTED: return "KA_ERR_UNSUPPORTED";
    case KA_ERR_WORKSPACE: return "KA_ERR_WORKSPACE";
    case KA_ERR_HIP: return "KA_ERR_HIP";
    default: return "KA_ERR_UNKNOWN";
  }
}

const char* ka_attn_last_error(void) { return g_last_error; }

}  // extern "C"
