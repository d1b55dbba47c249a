/*
 * kvq.h -- quantized-KV attention on AMD Instinct MI355X (gfx950).
 *
 * Scaled-dot-product attention over a per-layer KV cache held in affine group
 * quantization (4- or 8-bit codes, 64 values per group along head_dim, one
 * bf16 scale and one bf16 bias per group), for the decode and chunked-prefill
 * reads of a Gemma 4 text model.
 *
 * What the calls compute comes from the pages of the @mlx-bun/inference
 * 0.0.0-stage -> 1.0.0 diff on my.diffend.io:
 *   page 80, gemma4/model.ts, header notes: SDPA scale is 1.0 because q and k are
 *     RMS-normalised; full-attention layers have head_dim 512 and one KV head;
 *     sliding layers read a rotating cache whose reads own the window; KV-shared
 *     layers read a donor layer's cache;
 *   page 80, gemma4/model.ts, attentionTraining: keys and values are transposed
 *     to [B, H, L, D], appended to the layer's cache (cache.appendWindow), and
 *     the queries attend that read (read.attend(q, 1.0)); a sharer with no KV
 *     projection appends nothing and reads its donor;
 *   page 80, model.ts, decode / prompt phase declarations: decode is one new
 *     token per sequence; a prompt chunk is many tokens per sequence;
 *   page 78, gemma4-e4b.ts, Gemma4Layer and LAYERS: every cache is affine
 *     quantized with a width of 4 or 8 bits and a group of 64; sharers attend
 *     the last donor of their own attention type.
 * The pages give no quantization formula; this library uses, bit for bit:
 *     bias  = min(group) rounded down to bf16 (-0 read as +0)
 *     scale = ((max(group) - bias) / (2^bits - 1)) rounded up to bf16
 *     code  = clamp(rint((x - bias) / scale), 0, 2^bits - 1)   (0 when scale == 0)
 * with every step a single IEEE fp32 operation (round-to-nearest-even, no
 * fused multiply-add), and dequantizes as x = code * scale + bias.
 *
 * Conventions for every call:
 *   - Pointers are DEVICE pointers unless marked (host).  All memory is owned by
 *     the caller; the library allocates no device memory and keeps no pointer
 *     after a call returns.
 *   - Calls are asynchronous and ordered on `stream`.
 *   - Every argument that the host can see is validated before anything is
 *     launched; on a non-OK status nothing was launched and no output is
 *     touched.  kvq_last_error() then returns a message (thread-local).
 *   - Faults inside kernels surface at the next synchronisation of `stream`.
 *   - Sequence lengths live on the device and are read by the kernels; the
 *     host-side max_len only sizes the launch.  Every len[b] must be in
 *     [1, max_len] (prefill: [chunk, max_len]); otherwise results are
 *     unspecified, though every memory access stays inside the cache.
 *   - Calls that share one cache, workspace or output on one device must be
 *     ordered (same stream or events); concurrent calls on such buffers race.
 *   - Alignment: cache arrays, k and v 16 bytes; q 16 bytes; out 8 bytes; a
 *     workspace 16 bytes (checked; INVALID_ARGUMENT otherwise).  batch <= 32767, n_kv_heads <= 65535.
 *   - Precision: products accumulate in fp32 and out is rounded once to bf16.
 *     On quantized caches, decode reads (alone, shared or mixed), the decode
 *     step, and chunks of up to 16 query rows per KV head (rows = chunk *
 *     Hq/Hkv; alone or in a mixed launch, as for every chunk rule below)
 *     multiply the codes exactly and take any finite q and any cache
 *     the append wrote: q enters the fp16 MFMAs after a power of 2 per row and
 *     64-group (exact for every value within 2^-28 of the group's largest), and
 *     a step whose V scales reach 2^7 or V biases 2^15 runs its value product on
 *     bf16 operands split in two parts (about 16 bits) instead of fp16.  Chunks
 *     of 17..64 rows per KV head with head_dim 256 or 512 over more than 2048 keys
 *     normalize q per row the same way but dequantize K and V to fp16 (2^-11
 *     relative), so their values and scales must stay below 2^15 in magnitude
 *     (past that the output is not finite); chunks of more than 64 rows per KV
 *     head with head_dim 256 or 512 multiply the K codes exactly (q per row and
 *     128-column slice, the K scale and bias in fp32 and bf16 parts, as the
 *     decode read) and the V codes against p * v_scale in fp16, so their V
 *     scales must stay below 2^7 and V biases below 2^15 in magnitude.  Reads of
 *     bf16 caches multiply the stored values exactly, with q as bf16 and the
 *     softmax weights rounded to bf16 for the value product.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KVQ_OK = 0,
    KVQ_ERR_INVALID_ARGUMENT = 1, /* null pointer, bad count, Hq % Hkv != 0, ...      */
    KVQ_ERR_UNSUPPORTED = 2,      /* bits not 4/8 (or both 16), group != 64, head_dim not k*64 <= 512 */
    KVQ_ERR_CAPACITY = 3,         /* window > capacity, cache cannot hold the visible keys */
    KVQ_ERR_WORKSPACE = 4,        /* workspace smaller than the *_workspace_bytes query  */
    KVQ_ERR_HIP = 5               /* a HIP launch error                                   */
} kvq_status;

#define KVQ_GROUP_SIZE 64          /* values per quantization group along head_dim      */
#define KVQ_V_BLOCK 8              /* cache slots per V code block                      */
#define KVQ_MIN_CAPACITY 32        /* smallest cache capacity (one 32-key read step)     */
#define KVQ_MAX_SHARED_LAYERS 16   /* layers per kvq_shared_group                       */
#define KVQ_MAX_SHARED_GROUPS 4    /* groups per kvq_attn_decode_shared call             */
#define KVQ_STATIC_SCRATCH_BYTES (32 << 20)  /* device scratch of kvq_attn_decode_static  */

/*
 * (host) Descriptor of one layer's cache.  R = capacity slots; a token at
 * absolute position p lives in slot p mod R (a ring for sliding layers, a plain
 * array for full layers, which need R >= every length).  Layouts, with
 * B = batch, H = n_kv_heads, D = head_dim, G = D/64:
 *
 *   k_codes  uint32 [B][H][R][D*k_bits/32]   token-major: word w of a slot holds
 *            elements [w*k, (w+1)*k) of head_dim, k = 32/k_bits, element e at bits
 *            [k_bits*(e mod k), k_bits*(e mod k + 1))  (little-endian nibbles/bytes)
 *   v_codes  uint32 [B][H][R/8][D][v_bits/4]  blocked: block n holds slots 8n..8n+7;
 *            for each d its 8 codes are packed in v_bits/4 words, slot 8n+t at bits
 *            [v_bits*t, v_bits*(t+1)) of the block's v_bits bytes (little-endian)
 *   k_sb, v_sb  uint32 [B][H][R][G]  per slot and group: bf16 scale in bits 0..15,
 *            bf16 bias in bits 16..31
 *
 * A cache needs no clearing before its first append: reads fetch whole 32-key
 * steps and so touch slots past len that no append wrote, but such slots get
 * weight 0 and their contents (NaN bit patterns included) never reach out.
 *
 * The blocked V layout puts the 8 codes of one head_dim element for 8
 * consecutive slots in one place, which is what the value contraction over
 * keys reads; keys are read along head_dim, so K stays token-major.
 *
 * Unquantized bf16 cache (k_bits == v_bits == 16): page 80, gemma4/model.ts,
 * the note on cacheLayers, keeps the sliding layers' caches in bf16 under the
 * model's other KV scheme.  The same layouts hold the bf16 bit patterns of the
 * keys and values, rounded to nearest even from fp32, as 16-bit "codes" (K: 2
 * per word; V: a block's 8 values of one element in 4 words); k_sb and v_sb are
 * not used and may be NULL.  Every call takes such a cache; kvq_decode_step
 * rounds the step's token to bf16 where it would quantize it.
 *
 * Requirements: group_size == 64; head_dim a multiple of 64 from 64 to 512 (a bf16
 * cache: a multiple of 128); k_bits, v_bits in {4, 8}, or both 16; capacity a
 * multiple of 8 and at least KVQ_MIN_CAPACITY, with capacity * head_dim *
 * max(k_bits, v_bits) / 8 at most 8 GiB (the codes of one sequence and KV head
 * are addressed with 32-bit word offsets); 0 <= window <= capacity (0: full).
 * Chunk reads of more than 16 rows per KV head have kernels of their own at
 * head_dim 256 and 512 (the model's); at the other head_dims every read runs on
 * the decode kernel, which reads the keys once per 16-row tile.
 */
typedef struct {
    uint32_t *k_codes;
    uint32_t *v_codes;
    uint32_t *k_sb;
    uint32_t *v_sb;
    int32_t batch;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t group_size;
    int32_t k_bits;
    int32_t v_bits;
    int32_t capacity;
    int32_t window;
} kvq_cache;

/*
 * Quantize T new tokens per sequence and write them into the cache
 * (page 80, model.ts attentionTraining: cache.appendWindow(keys, values) before
 * the read; page 78, gemma4-e4b.ts Gemma4Layer.kv: affine width and group 64).
 *   k, v   fp32 [B][H][T][D], keys after norm and RoPE, values after norm
 *   T      (host) tokens per sequence, T >= 0 (0 is a no-op)
 *   pos0   int32 [B], absolute position of each sequence's first new token (>= 0)
 * Token t of sequence b goes to slot (pos0[b] + t) mod R.  With T > R only the
 * last R tokens are written.  Slots that this call does not write keep their
 * contents (a V block shared with untouched slots is read, merged and written).
 * Inputs must be finite with |x| <= 1e38; outside that the written codes are
 * unspecified.  A bf16 cache (k_bits == v_bits == 16) stores each value
 * rounded to the nearest bf16, ties to even, at the same slots.
 */
kvq_status kvq_append_quantize(const kvq_cache *cache,
                               const float *k, const float *v,
                               int32_t T, const int32_t *pos0,
                               hipStream_t stream);

/*
 * Several kvq_append_quantize calls in one launch, as one decode step writes
 * the new token of every layer that owns a cache (page 80, gemma4/model.ts
 * attentionTraining: appendWindow runs in each layer that owns its cache, and a
 * KV-shared layer reads the donor's cache without appending).
 *   items    n_items descriptors, 1 <= n_items <= KVQ_MAX_SHARED_GROUPS; item i
 *            has the arguments of one kvq_append_quantize call (T may differ)
 * Writes exactly what the separate calls would write.  Every item must name its
 * own cache (no two items may share k_codes or v_codes: KVQ_ERR_INVALID_ARGUMENT).
 * Quantized caches go in one kernel launch; a bf16 cache takes its own launch
 * after it.  Items are checked in order; on an error nothing is launched.
 */
typedef struct {
    const kvq_cache *cache;
    const float *k, *v;     /* fp32 [B][H][T][D] of this cache */
    int32_t T;
    const int32_t *pos0;    /* int32 [B] */
} kvq_append_item;

kvq_status kvq_append_quantize_multi(const kvq_append_item *items, int32_t n_items,
                                     hipStream_t stream);

/*
 * kvq_append_quantize with the norms and the rotation in front, in one kernel
 * (page 80, gemma4/model.ts attentionTraining: keys through kNorm and then the
 * rotary embedding at their cache positions, values through vNorm, then
 * appendWindow; header notes: the value norm has no learned scale, and the
 * rotation may cover only part of head_dim).
 *   k, v     fp32 [B][H][T][D], the projections before their norms (v may equal
 *            k, as where keys and values share one projection)
 *   T, pos0  as kvq_append_quantize: token t of sequence b sits at absolute
 *            position pos0[b] + t and goes to slot (pos0[b] + t) mod R
 *   k_weight fp32 [D], the key norm's weight, applied as given (a norm that
 *            scales by 1 + w takes 1 + w here); NULL for no weight
 *   eps      the norms' epsilon, finite and >= 0
 *   rope_cos, rope_sin  fp32 [rope_positions][rope_dims / 2]: the rotation
 *            table, indexed by absolute position (the pages do not give the
 *            angles; the caller's table fixes them)
 *   rope_dims  even, 0..D: the first rope_dims columns of each key rotate, column
 *            j paired with column j + rope_dims/2; 0 skips the rotation (tables
 *            may then be NULL)
 *   k_out, v_out  fp32 [B][H][T][D] or NULL: the normed (keys: rotated) rows of
 *            the tokens this call writes (the last min(T, R) of each sequence);
 *            other rows are left as they are
 * Per row of D values x (keys and values alike):
 *   r = 1 / sqrt(ss / D + eps), ss the sum of the squares, computed in fp64 and
 *       rounded once to fp32 (ss adds the squares pairwise over the row padded
 *       with zeros to a power of two);
 *   y_d = x_d * r (keys: then * k_weight[d]), each product rounded to fp32;
 *   keys, j < rope_dims/2, with c, s the table's entries j at the token's
 *   position: y_j' = y_j c - y_{j+n} s, y_{j+n}' = y_{j+n} c + y_j s
 *   (n = rope_dims/2; each product and sum rounded to fp32, no fused multiply-add);
 * then the rows are quantized (bf16 caches: rounded) and stored exactly as by
 * kvq_append_quantize.  Inputs must be finite with |x| <= 1e38; a row whose
 * ss / D + eps is 0 (all zeros with eps 0) has no norm and leaves unspecified
 * codes.  A position outside [0, rope_positions) reads the table's nearest
 * row (no memory outside the table is read); its rotated columns are then
 * unspecified.  Returns KVQ_ERR_INVALID_ARGUMENT for eps, rope_dims or the
 * tables out of range, or k_out / v_out not 16-byte aligned.
 */
kvq_status kvq_append_norm_quantize(const kvq_cache *cache,
                                    const float *k, const float *v,
                                    int32_t T, const int32_t *pos0,
                                    const float *k_weight, float eps,
                                    const float *rope_cos, const float *rope_sin,
                                    int32_t rope_dims, int32_t rope_positions,
                                    float *k_out, float *v_out,
                                    hipStream_t stream);

/*
 * One decode read: one query per sequence attends the cache
 * (page 80, model.ts decode declaration and attentionTraining read.attend(q, scale)).
 *   q      bf16 [B][Hq][D]; query head hq reads KV head hq / (Hq/Hkv)
 *   len    int32 [B], tokens in the cache including this step's; the query sits at
 *          p = len[b]-1 and sees positions max(0, p-W+1) .. p (W = window, 0: 0 .. p)
 *   max_len (host) upper bound of len[b]; sizes the launch
 *   scale  SDPA scale (1.0 for Gemma 4)
 *   out    bf16 [B][Hq][D] = softmax(scale * q.K^T) V, rounded to nearest even
 *   workspace  at least kvq_decode_workspace_bytes() bytes for the same arguments
 *          (may be NULL when that is 0); holds split partials, needs no clearing
 */
kvq_status kvq_attn_decode(const kvq_cache *cache,
                           const uint16_t *q, int32_t n_q_heads,
                           const int32_t *len, int32_t max_len, float scale,
                           uint16_t *out,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * kvq_attn_decode for callers that cannot allocate device memory and cannot
 * pass a workspace: code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation.  Same arguments, same kernels and the same result
 * as kvq_attn_decode, minus the workspace: the split partials go to a static
 * device array of KVQ_STATIC_SCRATCH_BYTES (32 MiB) inside this library, one
 * per device, allocated with the library's code on that device and held until
 * the process ends.  The call allocates nothing.  The stream must belong to
 * the current device.
 * A read whose partials need more than KVQ_STATIC_SCRATCH_BYTES (the size
 * kvq_decode_workspace_bytes reports for the same arguments; the split plan
 * aims at about 512 workgroups of 16 rows, so a head_dim-512 read needs at
 * most about 33 MB and most reads far less) returns KVQ_ERR_WORKSPACE and
 * launches nothing.
 * All calls on one device share that device's array: two of these calls that
 * overlap in time on one device (different streams, no ordering between them)
 * race and give wrong results; calls ordered on one stream are safe.  The
 * array needs no clearing between calls.
 */
kvq_status kvq_attn_decode_static(const kvq_cache *cache,
                                  const uint16_t *q, int32_t n_q_heads,
                                  const int32_t *len, int32_t max_len, float scale,
                                  uint16_t *out, hipStream_t stream);

/*
 * One decode step of a layer: append this step's token of every sequence and
 * read the cache with it (page 80, model.ts attentionTraining: appendWindow of
 * the new keys and values, then read.attend(q, scale); decode declaration: one
 * new token per sequence).  Equivalent to
 *   kvq_append_quantize(cache, k, v, 1, pos0 = len - 1) followed by
 *   kvq_attn_decode(cache, q, ..., len, ...),
 * with the same codes written bit for bit, in one attention launch (plus the
 * combine): the new token is quantized, written and attended from its
 * dequantized values by one more split per KV head while the other splits read
 * the older positions.
 *   k, v   fp32 [B][H][D], 16-byte aligned: the step's key (after norm and RoPE)
 *          and value of each sequence and KV head
 *   len    int32 [B], tokens including this one; it goes to slot (len[b]-1) mod R
 *   q, n_q_heads, max_len, scale, out  as for kvq_attn_decode
 *   workspace  at least kvq_decode_step_workspace_bytes() bytes; needs no clearing
 * k, v must be finite with |x| <= 1e38.
 */
kvq_status kvq_decode_step(const kvq_cache *cache,
                           const float *k, const float *v,
                           const uint16_t *q, int32_t n_q_heads,
                           const int32_t *len, int32_t max_len, float scale,
                           uint16_t *out,
                           void *workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * One chunked-prefill read (page 80, model.ts prompt / promptChunk: a whole chunk
 * of a prompt per sequence): the chunk's C tokens were appended first; query i of
 * sequence b sits at p = len[b] - C + i and sees max(0, p-W+1) .. p -- causal
 * inside the chunk, windowed across it.
 *   q    bf16 [B][Hq][C][D];  out bf16 [B][Hq][C][D]
 * Window layers need capacity >= window + C - 1 (the chunk must not overwrite a
 * key its first query still sees); full layers need capacity >= max_len.
 */
kvq_status kvq_attn_prefill_chunk(const kvq_cache *cache,
                                  const uint16_t *q, int32_t n_q_heads, int32_t chunk,
                                  const int32_t *len, int32_t max_len, float scale,
                                  uint16_t *out,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * (host) One cache read by the queries of n_layers KV-sharing layers
 * (page 80, model.ts header: KV-shared layers; page 78, gemma4-e4b.ts LAYERS:
 * sharers attend the last donor of their type, whose read is made once).
 *   q[l], out[l]  (host arrays of device pointers) bf16 [B][Hq][D] per layer
 *   len, max_len, scale  as for kvq_attn_decode, shared by the group's layers
 */
typedef struct {
    const kvq_cache *cache;
    int32_t n_layers;
    const uint16_t *const *q;
    uint16_t *const *out;
    int32_t n_q_heads;
    float scale;
    const int32_t *len;
    int32_t max_len;
} kvq_shared_group;

/*
 * Several shared groups, e.g. the sliding donor's sharers and the full donor's
 * sharers of one decode step, in one attention launch (plus one combine
 * launch).  Each layer's output equals a kvq_attn_decode of that layer alone.
 * 1 <= n_groups <= KVQ_MAX_SHARED_GROUPS.
 */
kvq_status kvq_attn_decode_shared(const kvq_shared_group *groups, int32_t n_groups,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * One decode step of several donors and their sharers (page 80, model.ts
 * header: KV-shared layers; attentionTraining: each donor appends its new keys
 * and values, then every layer reading that cache attends it; decode
 * declaration: one new token per sequence).  Equivalent to
 *   kvq_append_quantize(groups[i].cache, k[i], v[i], 1, pos0 = len_i - 1) for
 *   every group, followed by kvq_attn_decode_shared(groups, ...),
 * with the same codes written bit for bit, in one attention launch (plus the
 * combine): in each group the new token is quantized, written and attended
 * from its dequantized values by one more split per KV head, as in
 * kvq_decode_step.
 *   groups  as for kvq_attn_decode_shared; each group's len counts the new token,
 *           and no two groups may name the same cache (INVALID_ARGUMENT)
 *   k, v    (host arrays of n_groups device pointers) fp32 [B][H][D] of group i's
 *           cache, 16-byte aligned, finite with |x| <= 1e38: the keys (after
 *           norm and RoPE) and values of the token at position len[b] - 1
 *   workspace  at least kvq_decode_step_shared_workspace_bytes() bytes; needs no
 *           clearing
 */
kvq_status kvq_decode_step_shared(const kvq_shared_group *groups, int32_t n_groups,
                                  const float *const *k, const float *const *v,
                                  void *workspace, size_t workspace_bytes,
                                  hipStream_t stream);

/*
 * (host) One read of a mixed launch: like kvq_shared_group, plus the number of
 * queries per sequence.  chunk == 1 is a decode read by n_layers layers; chunk
 * > 1 is a short causal chunk (a speculative-verify window: query i of
 * sequence b sits at len[b] - chunk + i, as for kvq_attn_prefill_chunk) read
 * by one layer (n_layers == 1).
 *   q[l], out[l]  bf16 [B][Hq][chunk][D]
 * (page 80, model.ts: the decode and prompt phase declarations; reads of
 * different caches at different positions and phases share one grid.)
 */
typedef struct {
    const kvq_cache *cache;
    int32_t n_layers;
    const uint16_t *const *q;
    uint16_t *const *out;
    int32_t n_q_heads;
    int32_t chunk;
    float scale;
    const int32_t *len;
    int32_t max_len;
} kvq_read;

/*
 * Decode reads and short chunks of different caches in one attention launch
 * (plus one combine launch); each output equals that of the read alone
 * (kvq_attn_decode, or kvq_attn_prefill_chunk of the chunk) up to rounding.
 * 1 <= n_reads <= KVQ_MAX_SHARED_GROUPS.  A chunk runs on the decode kernel
 * (its rows, chunk x Hq/Hkv per KV head, read in 16-row tiles), except a
 * chunk of 17 to 64 rows per KV head over more than 2048 keys at head_dim 256
 * or 512 on a quantized cache: that one takes a launch of its own on the
 * short-chunk kernel, which holds all its rows per workgroup and so reads
 * each key once.
 */
kvq_status kvq_attn_mixed(const kvq_read *reads, int32_t n_reads,
                          void *workspace, size_t workspace_bytes,
                          hipStream_t stream);

/* (host) Workspace bytes for kvq_attn_mixed with these reads (SIZE_MAX when invalid). */
size_t kvq_mixed_workspace_bytes(const kvq_read *reads, int32_t n_reads);

/* (host) Workspace bytes for kvq_attn_decode_shared with these groups; for a
 * kvq_attn_decode call pass one group with n_layers = 1.  Returns 0 when the
 * call needs none, and SIZE_MAX when the arguments are invalid. */
size_t kvq_decode_workspace_bytes(const kvq_shared_group *groups, int32_t n_groups);

/* (host) Workspace bytes for kvq_decode_step with these arguments (SIZE_MAX when
 * they are invalid). */
size_t kvq_decode_step_workspace_bytes(const kvq_cache *cache, int32_t n_q_heads, int32_t max_len);

/* (host) Workspace bytes for kvq_decode_step_shared with these groups (SIZE_MAX
 * when they are invalid). */
size_t kvq_decode_step_shared_workspace_bytes(const kvq_shared_group *groups, int32_t n_groups);

/* (host) Workspace bytes for kvq_attn_prefill_chunk with these arguments. */
size_t kvq_prefill_workspace_bytes(const kvq_cache *cache, int32_t n_q_heads,
                                   int32_t chunk, int32_t max_len);

/*
 * (host) Measurement: arm two events for the next attention call made on this
 * thread (kvq_attn_decode, kvq_decode_step, kvq_attn_prefill_chunk,
 * kvq_attn_decode_shared or kvq_attn_mixed).  That call attaches `before` to
 * the start of its first read kernel (the split read, the prefill kernel or the
 * short-chunk kernel: not an append, a band copy or the combine of the split
 * partials) and `after` to the end of each read kernel it launches (the last
 * one stands), on the kernels themselves, so hipEventElapsedTime(before, after)
 * is the time from the first read kernel's start to the last one's end, without
 * the dispatch gaps around them.  Either event may be NULL.  The marks are used
 * by that one call and then dropped; a call that fails before its launch
 * records neither event.  Events are caller-created; nothing else changes.
 */
kvq_status kvq_mark_next_read(hipEvent_t before, hipEvent_t after);

/* (host) Message for the last non-OK status on this thread ("" if none). */
const char *kvq_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
