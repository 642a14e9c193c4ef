/*
 * pa_latent.h -- C ABI of the MI355X (gfx950) paged absorbed-MLA attention library.
 *
 * The operation is com.microsoft::PagedAttention with kv_cache_layout = "LATENT"
 * (absorbed multi-head latent attention, kv_num_heads = 1), as described on the
 * docs.rs page "onnx-runtime-ep-cuda src/kernels/paged_attention.rs", module
 * comment "LATENT semantics", and in PR #1978 ("native PagedAttention LATENT
 * kernel for GLM-5.2 dense MLA", section "What this adds"). It has two phases,
 * exposed as two entry points that must run in this order on one stream:
 *
 *   pa_latent_write      partial RoPE of each new latent key row, scattered in
 *                        place into the paged block cache at slot_mapping[t];
 *   pa_latent_attention  partial RoPE of each query head, then causal softmax
 *                        attention over the block_table-addressed latent prefix,
 *                        V = the leading v_head_size channels of the same row;
 *
 * and pa_latent_forward runs both in one call (the write's rows ride in the
 * read phase's first launch).
 *
 * Conventions for every entry point:
 *   - Device pointers are HIP device addresses on the current device; all tensors
 *     are dense row-major with the shapes given below (the page's kernel refuses
 *     strided inputs).
 *   - 16-bit tensors (query, key, key_cache, cos_cache, sin_cache, output) share
 *     one storage type, `dtype`. Index tensors are int32.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Calls are asynchronous: they enqueue kernels and return. They never
 *     synchronise, read device memory back, or allocate memory; launch geometry
 *     depends only on `attrs` and `dims`, so the calls can be captured in a HIP
 *     graph once the workspace is allocated.
 *   - Capture gate (docs.rs page, PagedCaptureSignature and capture_support;
 *     PR #1978 "Invariants held", capture/replay safe): a call made while its
 *     stream is being captured must have a warmed signature -- the same entry
 *     point with the same dtype, attributes, dims and device has completed
 *     once eagerly -- because the first eager call does the library's one-time
 *     host work (occupancy query, code-object load). Otherwise it returns
 *     PA_ERR_CAPTURE_NOT_WARMED and enqueues nothing. Replays of the captured
 *     work compute exactly what the eager calls compute.
 *   - Every argument check runs before the first launch: on any error nothing
 *     is enqueued. Errors return a pa_status and set a thread-local message read
 *     by pa_last_error().
 *   - The caller owns every buffer. The library allocates no device or host
 *     memory (op-side allocation is zero, PR #1978 "Invariants held").
 *   - Values the host cannot check without reading device memory are trusted
 *     preconditions, as on the pages (PR #1978 review, "Non-blocking
 *     observations"): cumulative_sequence_length[0] = 0, non-decreasing,
 *     last entry = token_count; past_seqlens[b] + new tokens of b <=
 *     max_blocks_per_seq * block_size; block_table entries of every block a
 *     sequence uses lie in [0, num_blocks); slot_mapping entries are -1 or in
 *     [0, num_blocks * block_size), distinct, and consistent with block_table;
 *     rotary_rows > largest position. Violating them gives unspecified
 *     results, but no access leaves the caller's buffers: block ids are
 *     clamped into [0, num_blocks), rotary positions into [0, rotary_rows),
 *     slots past the cache are skipped like -1, and the read phase plans its
 *     work from sequence bounds clamped into [0, token_count] and made
 *     non-decreasing and from past lengths clamped into
 *     [0, max_blocks_per_seq * block_size].
 */
#ifndef PA_LATENT_H
#define PA_LATENT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_LATENT_ABI_VERSION 3

typedef enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,    /* schema / geometry violation                      */
  PA_ERR_NOT_IMPLEMENTED = 2,     /* valid request the library does not implement     */
  PA_ERR_WORKSPACE_TOO_SMALL = 3, /* workspace_bytes < pa_latent_workspace_size(...)  */
  PA_ERR_DEVICE = 4,              /* a HIP runtime call failed                        */
  PA_ERR_CAPTURE_NOT_WARMED = 5   /* stream capture of a signature not yet run eagerly */
} pa_status;

/* Storage type of the 16-bit tensors; values are the ONNX TensorProto codes. */
typedef enum { PA_F16 = 10, PA_BF16 = 16 } pa_dtype;

/*
 * Node attributes, with the defaults the page's kernel factory applies
 * (docs.rs page, PagedAttentionFactory::create): v_head_size 0, rotary_offset 0,
 * do_rotary 0, rotary_interleaved 0, softcap 0, local_window_size -1, scale
 * absent. Passed by pointer; read only during the call.
 */
typedef struct {
  int32_t num_heads;          /* H >= 1 query heads (kv_num_heads is 1 by definition of LATENT) */
  int32_t head_size;          /* hs: latent row width = key_cache.shape[3]; hs % 8 == 0         */
  int32_t v_head_size;        /* 0 means hs; else 1 <= v_head_size <= hs                        */
  int32_t block_size;         /* key_cache.shape[1]: a power of two >= 16                      */
  int32_t do_rotary;          /* 0: no RoPE; nonzero: RoPE on [rotary_offset, +rotary_dim)     */
  int32_t rotary_interleaved; /* 0: pairs (d, d + rd/2); nonzero: pairs (2i, 2i+1)             */
  int32_t rotary_dim;         /* rd = 2 * cos_cache.shape[1]; rd % 16 == 0; ro + rd <= hs      */
  int32_t rotary_offset;      /* ro % 8 == 0                                                   */
  int32_t local_window_size;  /* < 0: off; W >= 0 keeps keys j with pos - j <= W               */
  float softcap;              /* <= 0: off; else scores become softcap * tanh(s / softcap)     */
  int32_t has_scale;          /* nonzero: use `scale`                                          */
  float scale;                /* explicit scale; required when v_head_size != head_size,       */
                              /* otherwise the default is 1 / sqrt(head_size)                  */
} pa_latent_attrs;

/* Host-known extents of the call's tensors. */
typedef struct {
  int64_t token_count;        /* T: rows of query / key / output / slot_mapping (>= 0)         */
  int32_t batch;              /* B >= 1: sequences = past_seqlens.shape[0]                     */
  int32_t max_blocks_per_seq; /* MB >= 1: block_table.shape[1]                                 */
  int64_t num_blocks;         /* NB >= 1: key_cache.shape[0]                                   */
  int64_t rotary_rows;        /* P: cos_cache.shape[0] (0 when do_rotary == 0)                 */
} pa_latent_dims;

/*
 * Write phase (docs.rs page, "LATENT semantics", write phase; device function
 * write_impl). For every new token t with slot = slot_mapping[t] >= 0:
 *   key_cache row `slot` (flat [NB*bs, hs] view) = RN(RoPE(key[t], pos(t)))
 * where b(t) is the first sequence with t < cumulative_sequence_length[b+1] and
 * pos(t) = past_seqlens[b] + t - cumulative_sequence_length[b]. RoPE computes in
 * float32 and only touches channels [rotary_offset, rotary_offset + rotary_dim);
 * RN rounds to nearest even. slot = -1 leaves the cache untouched.
 *
 *   key                        [T, hs]            dtype
 *   cos_cache, sin_cache       [P, rd/2]          dtype (may be NULL when do_rotary == 0)
 *   slot_mapping               [T]                int32
 *   cumulative_sequence_length [B + 1]            int32
 *   past_seqlens               [B]                int32
 *   key_cache                  [NB, bs, 1, hs]    dtype, updated in place
 *
 * Returns PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_NOT_IMPLEMENTED or PA_ERR_DEVICE.
 */
pa_status pa_latent_write(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                          const void* key, const void* cos_cache, const void* sin_cache,
                          const int32_t* slot_mapping, const int32_t* cumulative_sequence_length,
                          const int32_t* past_seqlens, void* key_cache, void* stream);

/*
 * Bytes of device workspace pa_latent_attention needs for these attrs/dims on
 * `device` (a HIP device ordinal). The op keeps transient compute scratch in
 * a workspace its caller manages, apart from the KV cache, whose only owner
 * is the caller's page authority (PR #1940 "PagedAttention v1 audit and MLA
 * oracle", third commit: the EP's scratch is EP-managed workspace, not a
 * second KV-cache authority; PR #1978 "Invariants held": no op-side
 * allocation). The workspace holds the on-device work schedule; when
 * head_size > 192 or v_head_size > 128, a RoPE'd copy of the query in the
 * attention kernel's fragment order; and the split-KV partial results
 * (float32 running max and denominator per row, and the piece's normalised
 * output row: bfloat16 for bfloat16 outputs, float32 for float16 ones).
 *
 * The size depends only on the arguments and the device's compute-unit count.
 * It is written to *bytes (0 on error) and the function returns a status like
 * every other entry point, so an unsupported geometry is reported with a
 * message rather than as a size of 0. Errors: PA_ERR_INVALID_ARGUMENT (NULL
 * bytes, or the checks pa_latent_attention makes on attrs/dims),
 * PA_ERR_NOT_IMPLEMENTED, PA_ERR_DEVICE (device query failed).
 */
pa_status pa_latent_workspace_size(const pa_latent_attrs* attrs, const pa_latent_dims* dims,
                                   pa_dtype dtype, int device, size_t* bytes);

/*
 * Read phase (docs.rs page, "LATENT semantics", read phase; device function
 * attn_impl; two-pass softmax form per PR #1940 "PagedAttention v1 audit and
 * MLA oracle"). For every new token t and head h:
 *   q      = RoPE(query[t, h*hs : (h+1)*hs], pos(t))
 *   keys   j in [0, pos(t)], and pos(t) - j <= local_window_size when that is >= 0
 *   row_j  = key_cache row block_table[b, j / bs] * bs + j % bs
 *   s_j    = scale * <q, row_j>;  s_j = softcap * tanh(s_j / softcap) when softcap > 0
 *   output[t, h*vhs : (h+1)*vhs] = RN( sum_j softmax(s)_j * row_j[0 : vhs] )
 * Must be ordered after pa_latent_write of the same step (it reads the rows
 * that call placed).
 *
 *   query                      [T, H * hs]        dtype
 *   key_cache                  [NB, bs, 1, hs]    dtype
 *   cos_cache, sin_cache       [P, rd/2]          dtype (may be NULL when do_rotary == 0)
 *   cumulative_sequence_length [B + 1]            int32
 *   past_seqlens               [B]                int32
 *   block_table                [B, MB]            int32 (entries past a sequence's last block
 *                                                 are never read; any value, e.g. -1)
 *   output                     [T, H * vhs]       dtype
 *   workspace                  workspace_bytes of device memory, 256-byte aligned,
 *                              >= pa_latent_workspace_size(...); contents on entry are
 *                              ignored, contents on exit are unspecified.
 *
 * Returns PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_NOT_IMPLEMENTED,
 * PA_ERR_WORKSPACE_TOO_SMALL or PA_ERR_DEVICE.
 */
pa_status pa_latent_attention(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                              const void* query, const void* key_cache, const void* cos_cache,
                              const void* sin_cache, const int32_t* cumulative_sequence_length,
                              const int32_t* past_seqlens, const int32_t* block_table, void* output,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Both phases in one call: pa_latent_write then pa_latent_attention on the
 * same stream, as the op's execute step enqueues its write kernel and then
 * its attention kernel for one set of inputs (docs.rs page, host function
 * execute; "LATENT semantics": the write phase places the new rows, the read
 * phase then attends over them). The results are those of the two calls
 * made in that order, bit for bit; the write's rows run in the read phase's
 * first launch (the on-device schedule, which reads none of what the write
 * stores), which saves one launch per step. Arguments are the union of the
 * two calls' (same meaning, layout and ownership; key_cache is updated in
 * place and then read), with the workspace of pa_latent_attention
 * (pa_latent_workspace_size). Every check of both calls runs before anything
 * is enqueued. Returns PA_OK, PA_ERR_INVALID_ARGUMENT, PA_ERR_NOT_IMPLEMENTED,
 * PA_ERR_WORKSPACE_TOO_SMALL, PA_ERR_CAPTURE_NOT_WARMED or PA_ERR_DEVICE.
 */
pa_status pa_latent_forward(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                            const void* query, const void* key, const void* cos_cache, const void* sin_cache,
                            const int32_t* slot_mapping, const int32_t* cumulative_sequence_length,
                            const int32_t* past_seqlens, const int32_t* block_table, void* key_cache,
                            void* output, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_latent_attention with the split-KV partition chosen by the caller:
 * split_kv != 0 is the automatic partition pa_latent_attention uses (work
 * spread evenly over the device's compute units, long key ranges split and
 * merged by a log-sum-exp combine); split_kv == 0 gives every query tile to a
 * single workgroup (no partial results, no combine). The two agree up to
 * rounding (float32 accumulation order; with bfloat16 outputs each piece's
 * output is rounded to bfloat16 before the combine); tests use this to check
 * the combine.
 */
pa_status pa_latent_attention_splits(const pa_latent_attrs* attrs, const pa_latent_dims* dims,
                                     pa_dtype dtype, const void* query, const void* key_cache,
                                     const void* cos_cache, const void* sin_cache,
                                     const int32_t* cumulative_sequence_length,
                                     const int32_t* past_seqlens, const int32_t* block_table,
                                     void* output, void* workspace, size_t workspace_bytes,
                                     int32_t split_kv, void* stream);

/*
 * pa_latent_attention for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * read phase, with the same kernels and results, but its workspace is a
 * static device array inside the library (64 MiB, one per device the library
 * runs on, held until the process ends) instead of a caller buffer. The call
 * itself allocates nothing. Arguments and errors are those of
 * pa_latent_attention; a call whose workspace (pa_latent_workspace_size)
 * exceeds 64 MiB returns PA_ERR_WORKSPACE_TOO_SMALL before any launch. Every
 * call on one device shares that device's array and leaves its contents
 * behind (nothing in it needs to start at zero): calls that overlap on one
 * device (different streams, or threads without ordering) race and give
 * undefined results.
 */
pa_status pa_latent_attention_noalloc(const pa_latent_attrs* attrs, const pa_latent_dims* dims,
                                      pa_dtype dtype, const void* query, const void* key_cache,
                                      const void* cos_cache, const void* sin_cache,
                                      const int32_t* cumulative_sequence_length,
                                      const int32_t* past_seqlens, const int32_t* block_table,
                                      void* output, void* stream);

/*
 * SEPARATE cache layout (grouped-query attention): the op's second dense mode,
 * with a key cache and a separate value cache of kv_num_heads heads each
 * (PR #1940 "PagedAttention v1 audit and MLA oracle", second commit: the
 * oracle's SEPARATE mode -- GQA, RoPE, softcap, local window -- over the same
 * block_table / slot_mapping addressing; third commit: num_heads must be a
 * multiple of kv_num_heads; PR #1978 review "Gates verified": the schema's
 * value and value_cache inputs). The pages print no kernel for it; where they
 * are silent this library takes: query head h uses key/value head
 * h / (num_heads / kv_num_heads) (consecutive heads form a group); RoPE, when
 * on, rotates channels [rotary_offset, rotary_offset + rotary_dim) of every
 * query head and every key head; value rows are stored unrotated; scale,
 * softcap, window and the remaining attributes behave as in the latent layout.
 * The attrs struct is the one above; kv_num_heads is passed beside it.
 * Built for head_size <= 128 and v_head_size <= head_size, v_head_size a
 * multiple of 8 (other valid sizes: PA_ERR_NOT_IMPLEMENTED).
 *
 * Write phase: for every token t with slot = slot_mapping[t] >= 0 and every
 * key/value head g,
 *   key_cache[slot, g]   = RN(RoPE(key[t, g*hs : (g+1)*hs], pos(t)))
 *   value_cache[slot, g] = value[t, g*vhs : (g+1)*vhs]
 *
 *   key                        [T, kvH * hs]      dtype
 *   value                      [T, kvH * vhs]     dtype
 *   key_cache                  [NB, bs, kvH, hs]  dtype, updated in place
 *   value_cache                [NB, bs, kvH, vhs] dtype, updated in place
 *   other arguments as in pa_latent_write.
 *
 * Read phase: for token t and head h in group g,
 *   q = RoPE(query[t, h*hs : (h+1)*hs], pos(t)); keys j as in pa_latent_attention;
 *   s_j = scale * <q, key_cache[row_j, g]> (softcap applied when on);
 *   output[t, h*vhs : (h+1)*vhs] = RN( sum_j softmax(s)_j * value_cache[row_j, g] )
 * with query [T, H * hs], output [T, H * vhs], the workspace sized by
 * pa_separate_workspace_size, and the other arguments as in
 * pa_latent_attention. Errors, ordering, ownership, capture gate (the
 * signature includes kv_num_heads) and trusted preconditions are those of the
 * latent entry points; kv_num_heads < 1 or num_heads % kv_num_heads != 0 is
 * PA_ERR_INVALID_ARGUMENT.
 */
pa_status pa_separate_write(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                            pa_dtype dtype, const void* key, const void* value, const void* cos_cache,
                            const void* sin_cache, const int32_t* slot_mapping,
                            const int32_t* cumulative_sequence_length, const int32_t* past_seqlens,
                            void* key_cache, void* value_cache, void* stream);

pa_status pa_separate_workspace_size(const pa_latent_attrs* attrs, int32_t kv_num_heads,
                                     const pa_latent_dims* dims, pa_dtype dtype, int device, size_t* bytes);

pa_status pa_separate_attention(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                                pa_dtype dtype, const void* query, const void* key_cache,
                                const void* value_cache, const void* cos_cache, const void* sin_cache,
                                const int32_t* cumulative_sequence_length, const int32_t* past_seqlens,
                                const int32_t* block_table, void* output, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * Both phases of the separate layout in one call: pa_separate_write then
 * pa_separate_attention on the same stream (docs.rs page, host function
 * execute), the write's key and value rows running in the read phase's first
 * launch, as in pa_latent_forward. Results bit-identical to the two calls in
 * that order; arguments are the union of theirs (key_cache and value_cache
 * updated in place, then read); every check of both runs before anything is
 * enqueued. Errors: those of pa_separate_attention and pa_separate_write.
 */
pa_status pa_separate_forward(const pa_latent_attrs* attrs, int32_t kv_num_heads, const pa_latent_dims* dims,
                              pa_dtype dtype, const void* query, const void* key, const void* value,
                              const void* cos_cache, const void* sin_cache, const int32_t* slot_mapping,
                              const int32_t* cumulative_sequence_length, const int32_t* past_seqlens,
                              const int32_t* block_table, void* key_cache, void* value_cache, void* output,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * Capture readiness of a signature on `device` (docs.rs page,
 * capture_support): *write_ready / *attention_ready are set to 1 when
 * pa_latent_write / pa_latent_attention with these dtype, attrs and dims have
 * completed eagerly on that device in this process (so they may be captured),
 * else 0. (pa_latent_forward is warmed by its own eager call; a capture of an
 * unwarmed one is refused with PA_ERR_CAPTURE_NOT_WARMED like the others.)
 * Returns PA_OK, or PA_ERR_INVALID_ARGUMENT for NULL arguments.
 */
pa_status pa_latent_capture_ready(const pa_latent_attrs* attrs, const pa_latent_dims* dims, pa_dtype dtype,
                                  int device, int32_t* write_ready, int32_t* attention_ready);

/* Measurement hook (not part of the method). `before` and `after` are
 * hipEvent_t handles created by the caller, or NULL. The next
 * pa_latent_attention / pa_latent_attention_splits / pa_separate_attention
 * call made on this thread
 * records `before` on its stream immediately before the launch of its
 * attention kernel and `after` immediately after it, so hipEventElapsedTime
 * of the pair is that kernel's duration without the schedule and combine
 * launches around it. The registration is consumed by that call (also when
 * it fails or launches nothing). Returns PA_OK. */
pa_status pa_latent_profile_next(void* before, void* after);

/* Message of the last failed call on this thread ("" after a successful call).
 * Valid until the next call into this library on the same thread. The op
 * reports every rejection as a typed error carrying a message that names the
 * offending attribute or input (docs.rs page, unsupported_reason and execute:
 * NotImplemented / KernelFailed with a reason string); the status code is the
 * type and this string the reason. */
const char* pa_last_error(void);

/* PA_LATENT_ABI_VERSION of the built library. */
int32_t pa_latent_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_LATENT_H */
