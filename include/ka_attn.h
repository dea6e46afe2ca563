/*
 * ka_attn.h -- C ABI of a grouped-query causal KV-cache attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The operation is the "states-form" attention of Karume's generation-context
 * path for Gemma 4 E2B: the rows of a prompt chunk, and later one decode row,
 * attend causally to the K / V rows a session keeps in its cache
 * (Karume v0.12.0 release notes, "Performance": the tiled states-form prefill
 * bullet and the two parallel-decode bullets; Karume v0.8.0 release notes,
 * "Features": the conversation-window bullet, which bounds the chunk at 768
 * rows and the cache at 131072 positions).  For a query row at absolute
 * position p, query head h and KV head g = h / (Hq / Hkv):
 *
 *     out[d] = sum_{j<=p} softmax_j(scale * q . k_g[j]) * v_g[j][d]
 *
 * Softmax rules (Karume v0.8.0 release notes, "Breaking Changes", the softmax
 * NaN bullet): a NaN among a row's visible scores makes that whole output row
 * NaN (the row max propagates NaN, no NaN is dropped); a NaN visible value
 * v[j][d] makes output dim d NaN, and an infinite one makes it infinite (NaN
 * with the other infinity, or when its weight is 0), as the row's own sum
 * gives it; masked keys carry weight exactly 0, so no key or value past a
 * row's position reaches its result -- a non-finite value at position j
 * inside a chunk reaches only the rows at j and after -- and no value at or
 * past the end of the chunk (or past a decode row) does.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - All pointers to tensors are DEVICE pointers (hipMalloc / torch memory on
 *    the current device); ka_attn_shape and ctx_len are HOST pointers.
 *  - The caller owns every buffer and the stream.  The library allocates no
 *    device memory: scratch space is the caller's `workspace`.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the default
 *    stream).  KA_OK means "validated and enqueued".
 *  - Every argument is validated on the host BEFORE anything is enqueued, so
 *    a rejected call leaves caches and outputs untouched.  The reason is kept
 *    per thread in ka_attn_last_error().
 *  - The library is stateless: positions are arguments.  Calls that touch the
 *    same cache must be ordered by the caller (one stream does that).
 *  - f32 means IEEE binary32; bf16 means the top 16 bits of binary32, written
 *    from f32 with round-to-nearest-even (NaN stays a quiet NaN).
 *
 * Tensor layouts (row-major, innermost last)
 * ------------------------------------------
 *   q, out (prefill)    f32 [B][R][Hq][D]     R = row_count of the chunk
 *   k_new, v_new        f32 [B][R][Hkv][D]
 *   q, out (decode)     f32 [B][Hq][D]
 *
 *   Caches: one K buffer and one V buffer, each ka_attn_cache_bytes() long,
 *   laid out in 16-byte vectors of E elements (E = 8 for bf16, 4 for f32) so
 *   that every kernel reads whole 16-byte vectors.  Element (b, g, j, d) --
 *   session b, KV head g, position j, dimension d -- lives at element index
 *
 *   K (f32, bf16):    ((((b*Hkv + g)*(C/64) + j/64)*(D/E) + d/E)*64 + j%64)*E + d%E
 *                     i.e. [B][Hkv][C/64][D/E][64][E]: per 64-position block,
 *                     E consecutive dims of 64 consecutive positions.
 *   V, f32:           (((b*Hkv + g)*(C/4) + j/4)*D + d)*4 + j%4
 *                     i.e. [B][Hkv][C/4][D][4]: per 4 positions, all dims.
 *   V, bf16:          ((((b*Hkv + g)*(C/32) + j/32)*4 + s)*D + d)*8 + t
 *                     with r = j%32, s = 2*(r/16) + (r%8)/4, t = r%4 + 4*((r%16)/8)
 *                     i.e. [B][Hkv][C/32][4][D][8]: each 32-position block in
 *                     four groups of 8 positions {16u+4h..16u+4h+3,
 *                     16u+8+4h..16u+8+4h+3}, group s = 2u + h.
 *
 *   int8-K caches (kv_dtype 2, KA_DTYPE_I8K): V as bf16 above; K as int8
 *   codes with one f32 scale per row (session, KV head, position), both in
 *   the K buffer: code (b, g, j, d) at BYTE index
 *                     (((b*Hkv + g)*(C/64) + j/64)*(D/16) + d/16)*64*16 + (j%64)*16 + d%16
 *   (the K layout above with E = 16), and the scale of row (b, g, j) as the
 *   f32 at byte B*Hkv*C*D + 4*((b*Hkv + g)*C + j).  Both buffers are
 *   ka_attn_cache_bytes() long (the V size; the K data use C*(D + 4) bytes per
 *   slab of it).  The append quantises each K row symmetrically (Karume
 *   v0.8.0 release notes, "Fixes": the activation-quantisation scale is amax
 *   times the f32 value of 1/127): s = f32(amax * f32(1/127)), code =
 *   round-half-even(x / s) limited to +-127 (IEEE f32 division); a row with
 *   a NaN gets s = NaN, one with an infinity s = inf, and rows whose s is 0
 *   or not finite get codes 0.  Attention quantises each query row (one
 *   head's D values) the same way and scores with the exact integer dot:
 *   score = scale * s_q * s_k * sum_d code_q[d] * code_k[d] (the pages' int8
 *   dot with i32 accumulation and an f32 epilogue, "Fixes": the dp4a bullet);
 *   V stays bf16.  The first int8 call on a device runs
 *   ka_attn_int8_self_test.
 *
 *   Cache contents beyond the rows appended so far are never read into a
 *   result (they may hold anything, NaN included).
 *
 * Limits: 1 <= Hkv, Hkv divides Hq, Hq <= 1024, D in {64, 128, 256}, C a
 * multiple of 64 with 64 <= C <= 131072, 1 <= batch <= 65536.  (With these
 * every size, index and launch grid the library forms stays far inside its
 * integer types; a shape beyond them is rejected as KA_ERR_OUT_OF_RANGE.)
 */
#ifndef KA_ATTN_H_
#define KA_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KA_ATTN_ABI_VERSION 1
#define KA_ATTN_MAX_CAPACITY 131072
#define KA_ATTN_MAX_Q_HEADS 1024
#define KA_ATTN_MAX_BATCH 65536

typedef enum ka_status {
  KA_OK = 0,
  KA_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad count, Hq % Hkv != 0, bad scale */
  KA_ERR_OUT_OF_RANGE = 2,     /* start + R > C, ctx < 1 or ctx > C, C, Hq or B too large */
  KA_ERR_UNSUPPORTED = 3,      /* head_dim or kv dtype not built                  */
  KA_ERR_WORKSPACE = 4,        /* workspace smaller than required                 */
  KA_ERR_HIP = 5               /* a HIP runtime error; text in ka_attn_last_error */
} ka_status;

typedef enum ka_dtype { KA_DTYPE_F32 = 0, KA_DTYPE_BF16 = 1, KA_DTYPE_I8K = 2 } ka_dtype;

typedef struct ka_attn_shape {
  int32_t batch;        /* B: independent sessions, each with its own cache rows */
  int32_t num_q_heads;  /* Hq                                                      */
  int32_t num_kv_heads; /* Hkv; query heads h*G .. h*G+G-1 share KV head h, G=Hq/Hkv */
  int32_t head_dim;     /* D in {64, 128, 256}                                     */
  int32_t capacity;     /* C: positions per session per KV head, multiple of 64    */
  int32_t kv_dtype;     /* ka_dtype of both caches                                 */
} ka_attn_shape;

/* Version of this ABI (KA_ATTN_ABI_VERSION of the built library). */
int32_t ka_attn_abi_version(void);

/* Bytes of ONE cache buffer (K or V) for shape s; 0 if s is invalid.  For
 * int8-K caches both buffers take the V size. */
size_t ka_attn_cache_bytes(const ka_attn_shape* s);

/*
 * KV append (the step that puts a chunk's rows into the session state before
 * they are attended; Karume v0.8.0 release notes, "Features": multi-turn
 * sessions continue the KV cache, and the context tracks the KV length).
 *
 * Writes rows k_new[b][i], v_new[b][i] (f32 [B][R][Hkv][D]) into cache
 * positions start_pos + i, i < row_count, of every session b: an exact copy
 * for f32 caches, round-to-nearest-even to bf16 for bf16 caches; on int8-K
 * caches K rows are quantised (see the int8-K layout above) and V rows
 * rounded to bf16.
 * row_count == 0 is a no-op.  Errors: KA_ERR_INVALID_ARGUMENT (null pointer,
 * row_count < 0, start_pos < 0), KA_ERR_OUT_OF_RANGE (start_pos + row_count
 * > C), KA_ERR_UNSUPPORTED, KA_ERR_HIP.
 */
ka_status ka_attn_append_kv(const ka_attn_shape* s, void* k_cache, void* v_cache,
                            const float* k_new, const float* v_new,
                            int32_t start_pos, int32_t row_count, void* stream);

/*
 * KV append with rotary position embedding of the new K rows.  The Karume
 * pages make the rotary tables a per-chunk host input: the host generates
 * the cos / sin rows of each chunk from the model's rope parameters (Karume
 * v0.8.0 release notes, "Features", the conversation-window bullet;
 * karume-gemma4-e2b model card, the context bullet).
 *
 * As ka_attn_append_kv, except that each new K row is first rotated:
 * rope_cos, rope_sin are f32 [row_count][D/2] device arrays (16-byte
 * aligned, like every f32 array here), row i holding the values for position
 * start_pos + i (shared by every session and KV head).  Dims d and d + D/2 form one pair (rotate-half pairing): for d < D/2
 *   k'[d]       = k[d] * cos[d] - k[d + D/2] * sin[d]
 *   k'[d + D/2] = k[d + D/2] * cos[d] + k[d] * sin[d]
 * evaluated in f32 as two rounded products and one rounded sum or difference
 * (no fused multiply-add), then stored like ka_attn_append_kv.  V rows are
 * stored as given.  Errors: those of ka_attn_append_kv; a null rope_cos or
 * rope_sin is KA_ERR_INVALID_ARGUMENT when row_count > 0.
 */
ka_status ka_attn_append_kv_rope(const ka_attn_shape* s, void* k_cache, void* v_cache,
                                 const float* k_new, const float* v_new,
                                 const float* rope_cos, const float* rope_sin,
                                 int32_t start_pos, int32_t row_count, void* stream);

/*
 * Rotary embedding of query rows (the same passages): x and y are f32
 * [B][row_count][Hq][D] device arrays (y may equal x for an in-place
 * rotation); row i of every session and head is rotated by rope_cos[i],
 * rope_sin[i] ([row_count][D/2]) exactly as ka_attn_append_kv_rope rotates
 * K rows.  row_count == 0 is a no-op.  Errors: KA_ERR_INVALID_ARGUMENT (null
 * pointer, row_count < 0), KA_ERR_UNSUPPORTED, KA_ERR_HIP.
 */
ka_status ka_attn_rope_rows(const ka_attn_shape* s, const float* x, float* y,
                            const float* rope_cos, const float* rope_sin, int32_t row_count,
                            void* stream);

/*
 * Workspace bytes that ka_attn_prefill_chunk needs for any chunk of at most
 * max_rows rows at any start position of shape s (0 if none is needed).
 */
size_t ka_attn_prefill_workspace_bytes(const ka_attn_shape* s, int32_t max_rows);

/*
 * Workspace bytes one ka_attn_prefill_chunk call with these arguments needs
 * (at most ka_attn_prefill_workspace_bytes(s, row_count); 0 if none is
 * needed or the arguments are invalid).  Host only.
 */
size_t ka_attn_prefill_workspace_need(const ka_attn_shape* s, int32_t start_pos,
                                      int32_t row_count);

/*
 * Chunked prefill (Karume v0.12.0 release notes, "Performance": the
 * states-form prefill on the GEMM tile skeleton, where the rows of a chunk
 * share each K / V row read; Karume v0.8.0 release notes, "Features": chunks
 * of up to 768 rows).
 *
 * Row i (i < row_count) of the chunk is at absolute position start_pos + i
 * and attends to cache positions 0 .. start_pos + i, which must already hold
 * appended rows.  Which kernel serves a chunk depends on its size (Karume
 * v0.12.0 release notes, "Docs": the plan-size geometry table for 1, 2-15
 * and 16 or more rows): on bf16 and int8-K caches a chunk of up to 15 rows may be
 * served by the split-context decode kernel, its (row, head) pairs taken as
 * columns with a causal limit each, when that is estimated to be faster;
 * otherwise, and on f32 caches, by the 128-column M-tile kernel.  Results
 * agree within the same tolerance either way.  q and out are f32 [B][R][Hq][D]; out may not alias q.
 * scale must be finite and > 0 (e.g. 1/sqrt(D)).  row_count == 0 is a no-op.
 * workspace: device scratch of at least
 * ka_attn_prefill_workspace_bytes(s, row_count) bytes (may be NULL when that
 * is 0).  Errors: KA_ERR_INVALID_ARGUMENT, KA_ERR_OUT_OF_RANGE (start_pos +
 * row_count > C), KA_ERR_UNSUPPORTED, KA_ERR_WORKSPACE, KA_ERR_HIP.
 */
ka_status ka_attn_prefill_chunk(const ka_attn_shape* s, const float* q,
                                const void* k_cache, const void* v_cache, float* out,
                                int32_t start_pos, int32_t row_count, float scale,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * A chunk's append and its prefill in one call: the same result, bit for
 * bit, as ka_attn_append_kv(s, k_cache, v_cache, k_new, v_new, start_pos,
 * row_count, stream) followed by ka_attn_prefill_chunk(s, q, k_cache, v_cache,
 * out, start_pos, row_count, scale, ...) -- the chunk's rows enter the state
 * before they are attended (Karume v0.8.0 release notes, "Features": sessions
 * continue the KV cache; v0.12.0, "Performance": the tiled states-form
 * prefill).  On bf16 caches, where the M-tile kernel serves the chunk, the
 * append kernel also stores the chunk's Q rows as bf16 of q * scale * log2(e),
 * rounded exactly as the prefill rounds its Q operands, in the workspace; the
 * prefill then reads those (half the bytes of f32 Q, and no conversion).
 * Arguments and layouts as for the two calls; out may not alias q.
 * workspace: device scratch of at least
 * ka_attn_append_prefill_workspace_bytes(s, row_count) bytes (may be NULL
 * when that is 0).  Errors: those of the two calls.
 */
ka_status ka_attn_append_prefill_chunk(const ka_attn_shape* s, const float* q,
                                       const float* k_new, const float* v_new, void* k_cache,
                                       void* v_cache, float* out, int32_t start_pos,
                                       int32_t row_count, float scale, void* workspace,
                                       size_t workspace_bytes, void* stream);

/*
 * Workspace bytes that ka_attn_append_prefill_chunk needs for any chunk of at
 * most max_rows rows at any start position of shape s (0 if none is needed):
 * ka_attn_prefill_workspace_bytes(s, max_rows) rounded up to 256, plus B *
 * max_rows * Hq * D * 2 on bf16 caches.
 */
size_t ka_attn_append_prefill_workspace_bytes(const ka_attn_shape* s, int32_t max_rows);

/*
 * Workspace bytes one ka_attn_append_prefill_chunk call with these arguments
 * needs (at most ka_attn_append_prefill_workspace_bytes(s, row_count); 0 if
 * none is needed or the arguments are invalid).  Host only.
 */
size_t ka_attn_append_prefill_workspace_need(const ka_attn_shape* s, int32_t start_pos,
                                             int32_t row_count);

/*
 * Workspace bytes that ka_attn_decode needs when no session's context length
 * exceeds max_ctx_len.
 */
size_t ka_attn_decode_workspace_bytes(const ka_attn_shape* s, int32_t max_ctx_len);

/*
 * Decode step (Karume v0.12.0 release notes, "Performance": the parallel QK
 * and PV reductions for one-row plans; Karume v0.8.0 release notes,
 * "Performance": the KV-axis parallel value accumulation).
 *
 * For each session b, the single query row q[b] (f32 [B][Hq][D]) sits at
 * position ctx_len[b] - 1 and attends to cache positions 0 .. ctx_len[b]-1
 * (so a step appends its own row first, then decodes).  ctx_len is a HOST
 * array of B entries, each 1 <= ctx_len[b] <= C.  out is f32 [B][Hq][D].
 * workspace: device scratch of at least
 * ka_attn_decode_workspace_bytes(s, max_b ctx_len[b]) bytes.  The result is
 * bitwise reproducible for the same inputs and shape.  Errors:
 * KA_ERR_INVALID_ARGUMENT, KA_ERR_OUT_OF_RANGE, KA_ERR_UNSUPPORTED,
 * KA_ERR_WORKSPACE, KA_ERR_HIP.
 */
ka_status ka_attn_decode(const ka_attn_shape* s, const float* q,
                         const void* k_cache, const void* v_cache, float* out,
                         const int32_t* ctx_len, float scale,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode step with its append (the same passages): for each session b, the
 * new K and V rows k_new[b], v_new[b] (f32 [B][Hkv][D]) are stored at cache
 * position pos[b], exactly as ka_attn_append_kv would store them (same
 * rounding, same bits), and the query row q[b] at that position attends to
 * cache positions 0 .. pos[b].  Equivalent to one ka_attn_append_kv per
 * session followed by ka_attn_decode with ctx_len[b] = pos[b] + 1, and bitwise
 * equal to it, in one attention launch on every cache dtype (the attention kernel writes the
 * row it uses).  pos is a HOST array of B entries, 0 <= pos[b] < C.  The
 * workspace is ka_attn_decode's for max_b pos[b] + 1.  k_new, v_new and q may
 * not overlap the caches or out.  Errors as ka_attn_decode.
 */
ka_status ka_attn_decode_step(const ka_attn_shape* s, const float* q, const float* k_new,
                              const float* v_new, void* k_cache, void* v_cache, float* out,
                              const int32_t* pos, float scale, void* workspace,
                              size_t workspace_bytes, void* stream);

/*
 * The decode step without any allocation and without a workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc.  Same
 * arguments, result and errors as ka_attn_decode_step, minus the workspace.
 *
 * The split partials live in a scratch array inside the library, one per
 * device (the current device at the call; stream must belong to it), of
 * ka_attn_decode_step_noalloc_max_bytes() bytes (8 MiB), held until the
 * process ends.  Its address on a device is looked up once, at the first
 * call on that device.  A call whose partials would not fit (only f32 caches
 * with several hundred (session, KV head) slabs) returns KA_ERR_WORKSPACE
 * before anything is enqueued.  The call allocates nothing and needs nothing
 * cleared: every partial it reads was written by the same call.  Every call
 * on one device shares that device's array: calls that may overlap in time
 * on one device (different streams without ordering between them) race and
 * must not be issued.  int8-K caches: the device self-test runs at the first
 * int8 call on a device (it copies its result to the host), so run
 * ka_attn_int8_self_test once before capturing such calls into a graph.
 */
size_t ka_attn_decode_step_noalloc_max_bytes(void);
ka_status ka_attn_decode_step_noalloc(const ka_attn_shape* s, const float* q,
                                      const float* k_new, const float* v_new, void* k_cache,
                                      void* v_cache, float* out, const int32_t* pos, float scale,
                                      void* stream);

/*
 * Ragged batches: sessions at different positions in one call (several
 * conversations served together, each continuing its own KV cache across
 * turns; Karume v0.8.0 release notes, "Features": the multi-turn chat session
 * and the per-run KV length).  start_pos and row_count are HOST arrays of B
 * entries; session b covers positions start_pos[b] .. start_pos[b] +
 * row_count[b] - 1 (row_count[b] == 0: the session takes no part).  Rows are
 * packed session by session: the rows of session b start at row
 * sum_{b' < b} row_count[b'] of every row array.  Each entry must satisfy
 * row_count[b] >= 0, start_pos[b] >= 0 and start_pos[b] + row_count[b] <= C.
 */

/*
 * Ragged KV append: k_new, v_new f32 [sum row_count][Hkv][D] (packed as
 * above) are stored at each session's positions as ka_attn_append_kv stores
 * them.  rope_cos / rope_sin: both NULL (no rotation) or f32 [sum row_count]
 * [D/2] packed the same way, each row holding its own position's values; the
 * K rows are then rotated as ka_attn_append_kv_rope rotates them.  All-zero
 * row counts are a no-op.  Errors: KA_ERR_INVALID_ARGUMENT (null pointer,
 * negative entry, only one of rope_cos / rope_sin), KA_ERR_OUT_OF_RANGE,
 * KA_ERR_UNSUPPORTED, KA_ERR_HIP.
 */
ka_status ka_attn_append_kv_ragged(const ka_attn_shape* s, void* k_cache, void* v_cache,
                                   const float* k_new, const float* v_new,
                                   const float* rope_cos, const float* rope_sin,
                                   const int32_t* start_pos, const int32_t* row_count,
                                   void* stream);

/*
 * Workspace bytes that ka_attn_prefill_ragged needs for any call whose row
 * counts add up to at most max_total_rows (0 if none is needed).
 */
size_t ka_attn_prefill_ragged_workspace_bytes(const ka_attn_shape* s, int64_t max_total_rows);

/*
 * Workspace bytes that one ka_attn_prefill_ragged call with these start_pos /
 * row_count host arrays needs (never more than the bound above for their
 * total; 0 if none is needed or the arguments are invalid).  Host only.
 */
size_t ka_attn_prefill_ragged_workspace_need(const ka_attn_shape* s, const int32_t* start_pos,
                                             const int32_t* row_count);

/*
 * Ragged chunked prefill: row i of session b (i < row_count[b]) is at
 * position start_pos[b] + i and attends to that session's cache positions
 * 0 .. start_pos[b] + i, exactly as ka_attn_prefill_chunk with that session's
 * start and row count.  q and out are f32 [sum row_count][Hq][D], packed as
 * above; out may not alias q.  The sessions' tiles share each launch, so
 * short chunks of many sessions fill the GPU together.  Every session runs
 * on the M-tile kernel (on bf16 and int8-K caches the few-row form of
 * ka_attn_prefill_chunk is not used here).  workspace: device scratch of at
 * least ka_attn_prefill_ragged_workspace_bytes(s, sum row_count) bytes.
 * Errors: those of ka_attn_prefill_chunk, per entry.
 */
ka_status ka_attn_prefill_ragged(const ka_attn_shape* s, const float* q,
                                 const void* k_cache, const void* v_cache, float* out,
                                 const int32_t* start_pos, const int32_t* row_count, float scale,
                                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Memory a session window costs before it is allocated (Karume v0.8.0
 * release notes, "Features": the conversation-window bullet's session memory
 * estimate for a capacity and chunk length; "Breaking Changes": the estimate
 * counts the attention's transient buffers).  For shape s (its capacity is
 * the window) and chunks of at most max_chunk_rows rows:
 *   cache_bytes              K and V caches (2 x ka_attn_cache_bytes)
 *   prefill_workspace_bytes  ka_attn_prefill_workspace_bytes(s, max_chunk_rows)
 *   decode_workspace_bytes   ka_attn_decode_workspace_bytes(s, C)
 *   chunk_io_bytes           one chunk's f32 q, out, k_new and v_new rows
 *   total_bytes              cache + the larger workspace (prefill and decode
 *                            calls can share one) + chunk_io_bytes
 * Errors: KA_ERR_INVALID_ARGUMENT (m NULL), KA_ERR_OUT_OF_RANGE
 * (max_chunk_rows outside 1 .. C), and the shape errors.
 */
typedef struct ka_attn_memory {
  size_t cache_bytes;
  size_t prefill_workspace_bytes;
  size_t decode_workspace_bytes;
  size_t chunk_io_bytes;
  size_t total_bytes;
} ka_attn_memory;
ka_status ka_attn_session_memory(const ka_attn_shape* s, int32_t max_chunk_rows,
                                 ka_attn_memory* m);

/*
 * Cache re-allocation to another window ("Gemma 4 E2B · WebGPU Kernels",
 * "Top-bar Context Control": a context cap change re-allocates the on-device
 * KV cache):
 * copies cache positions 0 .. rows - 1 of every session and KV head from
 * caches of shape src to caches of shape dst, which may differ from src in
 * capacity only.  rows <= both capacities; positions at or past rows in dst
 * are left undefined.  The copy is asynchronous on stream; the two cache
 * pairs must not overlap.  Errors: KA_ERR_INVALID_ARGUMENT (shapes differ in
 * more than capacity, rows < 0, null pointer, overlap),
 * KA_ERR_OUT_OF_RANGE (rows above a capacity), the shape errors, KA_ERR_HIP.
 */
ka_status ka_attn_cache_resize(const ka_attn_shape* src, const void* src_k, const void* src_v,
                               const ka_attn_shape* dst, void* dst_k, void* dst_v, int32_t rows,
                               void* stream);

/*
 * Device self-test of the int8 scores (Karume v0.8.0 release notes, "Fixes":
 * the int8 dot is not taken on faith; a canary checks the instruction and its
 * emulation against a known answer at first use, and the library fails
 * loudly when they are not sane).  On the current device, one wave
 * multiplies fixed int8 patterns (16 x 64 by 64 x 16, and 32 x 32 by
 * 32 x 32) with each int8 MFMA instruction the int8-K kernels use, in their
 * lane layouts, and with plain integer arithmetic; all must equal the exact
 * products.  It runs once per
 * device (synchronising the device that once; call it before capturing a
 * graph) and the outcome is kept.  Every int8-K attention call runs it first.
 * Returns KA_OK, or KA_ERR_UNSUPPORTED (int8-K attention calls then fail the
 * same way; the text names what disagreed), or KA_ERR_HIP.
 */
ka_status ka_attn_int8_self_test(void);

/* Static name of a status code ("KA_OK", ...). */
const char* ka_attn_status_string(int32_t status);

/* Reason for the last non-KA_OK status returned on this thread ("" if none). */
const char* ka_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KA_ATTN_H_ */
