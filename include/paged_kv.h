/*
 * paged_kv.h — C ABI of libpagedkv: attention over a paged KV cache for one
 * continuous-batching step, on AMD Instinct MI355X (gfx950).
 *
 * Sources for what the calls compute (cited by page title and section):
 *  - "AI Infra入门干货总结：大模型是如何高效推理的", section "Paged Attention":
 *    the cache layout [num_layers, 2, num_blocks, block_size, num_kv_heads,
 *    head_dim], the per-request block_table [max_num_reqs,
 *    max_num_blocks_per_req] of physical block ids, and slot_mapping, which
 *    tells the kernel where to store each new token's K/V, with
 *    slot = block * block_size + offset.
 *  - Same page, section "连续批处理 (Continuous Batching)": num_computed_tokens
 *    counts the tokens of a request already in the cache.
 *  - Same page, section "LLM 推理全流程", "Attention (FlashAttention)": Q is
 *    [query_lens, num_heads, head_dim], K/V are read from the paged cache as
 *    [seq_lens, num_kv_heads, head_dim], and a group of query heads shares one
 *    KV head by index (GQA); attention is computed tile by tile with an online
 *    softmax.
 *  - lpnh.cn/news/2669538, section 2.1: attention is
 *    softmax(q k^T * scale + mask) v.
 *
 * Conventions shared by every call:
 *  - block_size is fixed at 16 tokens.
 *  - Element types: PKV_F32 (IEEE float32) or PKV_BF16 (bfloat16). q, k, v,
 *    the cache and out all use the same type.
 *  - One layer of the cache is passed: kv_cache_layer points at
 *    [2][num_blocks][16][num_kv_heads][head_dim] elements (K at index 0, V at
 *    index 1), row-major, contiguous.
 *  - All array arguments are DEVICE pointers owned by the caller, except where
 *    a call says "host".  Tensors must be contiguous; q, k, v, out and the
 *    cache must be 16-byte aligned.
 *  - head_dim must be 64 or 128; num_q_heads must be a multiple of
 *    num_kv_heads with num_q_heads / num_kv_heads <= 16; paged_attention
 *    takes at most 240 kv heads.
 *  - stream is a hipStream_t (NULL = the legacy default stream).  Work is only
 *    enqueued: the calls return before the GPU finishes, never synchronise,
 *    never allocate or free device memory.  The caller keeps every buffer alive until
 *    the stream reaches that point.
 *  - The calls may be made from several host threads at once.  The only
 *    process-wide state is a per-kernel cache of the occupancy the HIP runtime
 *    reports (filled on first use with the same value by every caller), one
 *    library stream per device (created on first use, default priority; see
 *    paged_attention_int8) and the per-thread error detail string.  Two calls
 *    that share a workspace must be ordered on one stream.
 *  - Errors are returned as a pkv_status, never thrown.  Argument errors are
 *    detected on the host before anything is enqueued.  Bad *contents* of
 *    device metadata (inconsistent lengths, out-of-range block ids or slots)
 *    are detected on the device: the affected output rows are written as NaN
 *    (cache writes are skipped) and a bit is set in a device error word that
 *    pkv_read_device_error() returns.
 */
#ifndef PAGED_KV_H_
#define PAGED_KV_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_BLOCK_SIZE 16

typedef enum { PKV_F32 = 0, PKV_BF16 = 1 } pkv_dtype;

typedef enum {
  PKV_OK = 0,
  PKV_ERR_NULL = 1,       /* a required pointer is NULL */
  PKV_ERR_DIMS = 2,       /* a size is negative, zero where it may not be, or unsupported */
  PKV_ERR_DTYPE = 3,      /* dtype is not a pkv_dtype */
  PKV_ERR_WORKSPACE = 4,  /* workspace smaller than paged_attention_workspace_size() */
  PKV_ERR_LAUNCH = 5,     /* the HIP runtime refused a launch (see pkv_last_error_detail) */
  PKV_ERR_METADATA = 6,   /* host validator: metadata contents are inconsistent */
  PKV_ERR_ALIGN = 7       /* a pointer is not 16-byte aligned */
} pkv_status;

/* Bits of the device error word. */
#define PKV_DEVERR_SEQ_LEN     0x1  /* seq_lens[r] != num_computed_tokens[r] + query_len, or a length < 0 */
#define PKV_DEVERR_LIMITS      0x2  /* query_len > max_query_len, seq_len > max_seq_len, or
                                       seq_len > 16 * max_blocks_per_req */
#define PKV_DEVERR_QSL         0x4  /* query_start_loc not non-decreasing from 0, or past num_tokens */
#define PKV_DEVERR_BLOCK_ID    0x8  /* a block_table entry read is outside [0, num_blocks) */
#define PKV_DEVERR_SLOT        0x10 /* a slot_mapping entry is < -1 or >= 16 * num_blocks */
#define PKV_DEVERR_CAPACITY    0x20 /* the workspace was too small for this step's split-KV partials */
#define PKV_DEVERR_POSITION    0x40 /* a position given to paged_kv_write_rope is outside [0, max_position) */

/*
 * paged_kv_write — store the step's new K/V in the cache (a "slot_mapping"
 * scatter: "AI Infra入门干货总结", section "Paged Attention").
 *
 *   k, v            device, [num_tokens][num_kv_heads][head_dim], dtype.
 *   slot_mapping    device, int64 [num_tokens].  Token t goes to block
 *                   slot / 16, offset slot % 16.  -1 marks a padding token,
 *                   which is skipped.  Any other value outside
 *                   [0, 16 * num_blocks) is skipped and sets PKV_DEVERR_SLOT.
 *                   Two tokens must not share a slot (the result would be
 *                   either token's data).
 *   kv_cache_layer  device, [2][num_blocks][16][num_kv_heads][head_dim], dtype.
 *                   Only the addressed slots change; the bits are copied
 *                   unchanged.
 *   device_error    device int32, or NULL.  When non-NULL, PKV_DEVERR_SLOT is
 *                   OR-ed into it on a bad slot.
 *   num_tokens      >= 0 (0 enqueues nothing).
 * Returns PKV_OK or an argument error.
 */
int paged_kv_write(const void* k, const void* v, const int64_t* slot_mapping,
                   void* kv_cache_layer, int64_t num_tokens, int32_t num_blocks,
                   int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                   int32_t* device_error, void* stream);

/*
 * paged_attention — attention of one step's query tokens over the paged cache.
 *
 * Request r owns query rows [query_start_loc[r], query_start_loc[r+1]) of q
 * and out.  Its query_len = query_start_loc[r+1] - query_start_loc[r] may be
 * 0 (nothing is computed), 1 (a decode) or more (a prefill chunk).  Its
 * seq_len must equal num_computed_tokens[r] + query_len: the step's new
 * tokens are already in the cache (paged_kv_write runs first on the same
 * stream).  Query row i of the request sits at absolute position
 * num_computed_tokens[r] + i and attends to the request's cached tokens
 * 0 .. that position (causal within the chunk, full over the cached prefix).
 * Token t of the request is read from physical block block_table[r][t / 16],
 * offset t % 16.  Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *
 *   out                  device, [num_tokens][num_q_heads][head_dim], dtype (written).
 *                        Rows past query_start_loc[num_reqs] are not written.
 *   q                    device, [num_tokens][num_q_heads][head_dim], dtype.
 *   kv_cache_layer       device, [2][num_blocks][16][num_kv_heads][head_dim], dtype.
 *   block_table          device, int32 [num_reqs][max_blocks_per_req].  Only the
 *                        first ceil(seq_len / 16) entries of a row are read.
 *   seq_lens             device, int32 [num_reqs].
 *   query_start_loc      device, int32 [num_reqs + 1], non-decreasing, [0] == 0,
 *                        [num_reqs] <= num_tokens.
 *   num_computed_tokens  device, int32 [num_reqs].
 *   scale                multiplies q.k before the softmax (usually 1/sqrt(head_dim)).
 *   max_query_len        host bound on every query_len (sizes the prefill grid).
 *   max_seq_len          host bound on every seq_len (sizes the split-KV grid).
 *   workspace            device scratch of workspace_bytes >=
 *                        paged_attention_workspace_size(...) bytes, 256-byte
 *                        aligned.  Holds the device error word (cleared by each
 *                        call), work lists and split-KV partials.
 * Slots of the cache that no request reads (the tail of a request's last
 * block, unused blocks) may hold anything, NaN included; they never reach out.
 * Results are deterministic: the same inputs give the same bits, whatever the
 * other requests of the batch and their order.
 * Returns PKV_OK or an argument error.
 */
int paged_attention(void* out, const void* q, const void* kv_cache_layer,
                    const int32_t* block_table, const int32_t* seq_lens,
                    const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                    float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                    int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                    int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                    int32_t dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * paged_attention_profiled — paged_attention, plus hipEvent_t records around
 * each internal phase, for measurement tools that time a kernel on the
 * library's own stream.  phase_events points at 2 * PKV_NUM_PHASES event
 * handles (hipEvent_t, created by the caller; any entry may be NULL):
 * entry 2*p is recorded just before phase p is enqueued and 2*p+1 just after.
 * A phase that has no work for the step still records both events.  The
 * computation and its results are exactly those of paged_attention.
 */
#define PKV_PHASE_PLAN 0     /* metadata checks and work lists */
#define PKV_PHASE_PREFILL 1  /* causal chunked prefill (bf16 MFMA) */
#define PKV_PHASE_ROWS 2     /* decode rows and split-KV partitions */
#define PKV_PHASE_REDUCE 3   /* split-KV merge */
#define PKV_NUM_PHASES 4
int paged_attention_profiled(void* out, const void* q, const void* kv_cache_layer,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                             float scale, int32_t num_reqs, int64_t num_tokens,
                             int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t num_blocks, int32_t max_blocks_per_req,
                             int32_t max_query_len, int32_t max_seq_len, int32_t dtype,
                             void* workspace, size_t workspace_bytes, void* stream,
                             void* const* phase_events);

/*
 * paged_attention_noalloc — paged_attention for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same computation and results, with the
 * workspace taken from a static device array of PKV_NOALLOC_SCRATCH_BYTES
 * that the library holds on every GPU it runs on until the process ends.
 * Arguments are those of paged_attention without workspace / workspace_bytes;
 * the caller still owns q, out, the cache and the metadata.  It calls no
 * hipMalloc, hipFree or allocating library routine.
 *   device_error    device int32, or NULL.  When non-NULL, the step's
 *                   PKV_DEVERR_* bits are OR-ed into it (the scratch is not
 *                   visible to the caller, so pkv_read_device_error does not
 *                   apply).
 * Returns PKV_ERR_WORKSPACE, before anything is enqueued, when
 * paged_attention_workspace_size for these bounds would exceed the scratch.
 * Every call on one GPU uses that GPU's one scratch array, which keeps the
 * last call's contents (each call rebuilds what it reads): calls that may
 * overlap on one GPU (several streams or threads) race and must be ordered
 * by the caller.
 */
#define PKV_NOALLOC_SCRATCH_BYTES (128u << 20)
int paged_attention_noalloc(void* out, const void* q, const void* kv_cache_layer,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                            float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                            int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                            int32_t dtype, int32_t* device_error, void* stream);

/*
 * paged_attention_workspace_size — bytes of workspace paged_attention needs
 * for these bounds (same meaning as its arguments).  Returns 0 for invalid
 * sizes.  Pure host function.
 */
size_t paged_attention_workspace_size(int32_t num_reqs, int64_t num_tokens,
                                      int32_t num_q_heads, int32_t head_dim,
                                      int32_t max_query_len, int32_t max_seq_len);

/*
 * pkv_read_device_error — wait for `stream`, then return the device error word
 * of the last paged_attention call that used `workspace` (0 = no error, else
 * PKV_DEVERR_* bits), or -1 if the copy failed.  This call synchronises.
 */
int32_t pkv_read_device_error(const void* workspace, void* stream);

/*
 * pkv_validate_metadata_host — check a step's metadata on the host, with no
 * HIP call.  All pointers are HOST arrays with the shapes paged_attention
 * uses; slot_mapping (int64 [num_tokens]) may be NULL.  Checks the
 * query_start_loc, seq_len and limit rules, that every block id a request
 * reads is in [0, num_blocks), that every slot is -1 or in
 * [0, 16 * num_blocks), and that no two tokens share a slot.
 * Returns PKV_OK or PKV_ERR_METADATA / PKV_ERR_NULL / PKV_ERR_DIMS
 * (pkv_last_error_detail() says which request or token).
 */
int pkv_validate_metadata_host(const int32_t* block_table, const int32_t* seq_lens,
                               const int32_t* query_start_loc,
                               const int32_t* num_computed_tokens, const int64_t* slot_mapping,
                               int32_t num_reqs, int64_t num_tokens, int32_t num_blocks,
                               int32_t max_blocks_per_req, int32_t max_query_len,
                               int32_t max_seq_len);

/*
 * paged_kv_write_rope — paged_kv_write with the rotary position embedding
 * applied to K on its way into the cache, and optionally to q in place
 * ("AI Infra入门干货总结", section "LLM 推理全流程" / "RoPE": positions are
 * rotation angles read from a precomputed cos_sin_cache of shape
 * [max_position_embeddings, rotary_dim]).
 *
 *   q               device, [num_tokens][num_q_heads][head_dim], dtype, or
 *                   NULL.  When given, every row is rotated in place.
 *   k, v            device, [num_tokens][num_kv_heads][head_dim], dtype
 *                   (not modified).
 *   positions       device, int64 [num_tokens]: absolute position of each
 *                   token in its sequence.  A token whose position is
 *                   outside [0, max_position) is left alone entirely (no q
 *                   rotation, no cache write) and sets PKV_DEVERR_POSITION.
 *   cos_sin_cache   device, float32 [max_position][rotary_dim]: row p holds
 *                   cos of the rotary_dim/2 angles of position p, then their
 *                   sin.
 *   rotary_dim      even, 2 .. head_dim; dims from rotary_dim on are not
 *                   rotated.
 *   is_neox         1: angle i rotates the pair (i, i + rotary_dim/2);
 *                   0: the pair (2i, 2i+1).  x' = x cos - y sin,
 *                   y' = y cos + x sin, in fp32, rounded to dtype (nearest
 *                   even).
 *   slot_mapping, kv_cache_layer, num_blocks, num_kv_heads, head_dim, dtype,
 *   device_error    as for paged_kv_write (V is copied unchanged; slot -1
 *                   skips the cache write but q is still rotated).
 * Returns PKV_OK or an argument error; enqueued on `stream`.
 */
int paged_kv_write_rope(void* q, const void* k, const void* v, const int64_t* positions,
                        const float* cos_sin_cache, int32_t max_position, int32_t rotary_dim,
                        int32_t is_neox, const int64_t* slot_mapping, void* kv_cache_layer,
                        int64_t num_tokens, int32_t num_q_heads, int32_t num_blocks,
                        int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                        int32_t* device_error, void* stream);

/*
 * INT8 KV cache (online quantisation of the cache as it is written and
 * dequantisation as it is read: lpnh.cn/news/2436702, section 4.2, "KV
 * Cache 量化").  The cache of one layer is
 *   kv_cache_layer  int8 [2][num_blocks][16][num_kv_heads][head_dim] codes,
 *   kv_scales       float32 [2][num_blocks][num_kv_heads][16] scales (a kv
 *                   head's 16 scales of a block are contiguous; the scale of
 *                   slot (block b, offset o), head h is [kv][b][h][o]),
 * value = code * scale.  Each (token, K or V, kv head) row of head_dim
 * values is quantised on its own: scale = max|x| / 127, code =
 * round-half-even(x / scale) clamped to [-127, 127], both divisions IEEE
 * float32; an all-zero row has scale 0 and codes 0.  Half the bytes of a
 * bf16 cache, plus 4 bytes per row.
 *
 * paged_kv_write_int8 — quantise and store the step's new K/V (k, v in
 *   dtype, [num_tokens][num_kv_heads][head_dim]) at slot_mapping, like
 *   paged_kv_write; codes and scales of the addressed slots change.
 * paged_attention_int8 — paged_attention over such a cache: the keys and
 *   values are the dequantised rows; q and out are in dtype (bf16 or fp32).
 *   With bf16 q and head_dim 128, prefill chunks run on the matrix-core
 *   prefill kernel, which dequantises each streamed tile in LDS (code *
 *   scale in float32, rounded to bf16) before both products.  Every other
 *   row (decode rows, split-KV partitions of 1024 tokens, and
 *   prefill rows of other dtypes or head sizes) runs on a row kernel: with
 *   bf16 q all G query heads of a kv head share 16x16 matrix-core tiles over
 *   the exact integer codes, the scales entering in float32 (p * v_scale is
 *   rounded to bf16); with fp32 q a VALU kernel works in float32.
 *   workspace_bytes beyond paged_attention_workspace_size() is a staging
 *   area: when the step's prefill chunks (bf16 q, head_dim 128) read at most
 *   as many cache blocks as fit there (paged_attention_staging_bytes), each
 *   of those blocks is dequantised once into a bf16 block of the staging area
 *   (code * scale in float32, rounded to bf16: the values the prefill kernel
 *   forms in LDS, so results are the same bit for bit) and the prefill reads
 *   the staged blocks instead of dequantising every tile it streams.  With no
 *   extra workspace, or a step that does not fit, nothing changes.
 *   phase_events as for paged_attention_profiled, or NULL.  With NULL and
 *   no staging area, the prefill kernel of a step that has prefill chunks
 *   runs on a library stream beside `stream` (which waits for it through
 *   events created and released by the call, so `stream` still orders
 *   everything): the row kernels take the CUs that the prefill's last
 *   workgroups leave free.  With a staging area, or with phase events, every
 *   kernel runs on `stream`, one after the other.
 * Other arguments, the workspace and the error conventions are those of
 * paged_kv_write / paged_attention.
 */
/*
 * paged_attention_staging_bytes — workspace bytes to add to
 * paged_attention_workspace_size() so that paged_attention_int8 / _fp8 stage
 * the prefill of any step whose prefill requests read at most prefill_blocks
 * cache blocks in all (the sum over the prefill requests of
 * ceil(seq_len / 16)); num_reqs and max_blocks_per_req as in the call.
 * Returns 0 for prefill_blocks == 0 or invalid sizes.  Pure host function.
 */
size_t paged_attention_staging_bytes(int32_t num_reqs, int32_t max_blocks_per_req, int32_t num_kv_heads,
                                     int32_t head_dim, int64_t prefill_blocks);
int paged_kv_write_int8(const void* k, const void* v, const int64_t* slot_mapping, void* kv_cache_layer,
                        float* kv_scales, int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                        int32_t head_dim, int32_t dtype, int32_t* device_error, void* stream);
int paged_attention_int8(void* out, const void* q, const void* kv_cache_layer, const float* kv_scales,
                         const int32_t* block_table, const int32_t* seq_lens,
                         const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                         float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                         int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                         int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                         int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                         void* const* phase_events);

/*
 * FP8 KV cache: the INT8 cache's layout and per-(token, K or V, kv head)
 * scales (online KV-cache quantisation, lpnh.cn/news/2436702, section 4.2),
 * with codes in the OCP 8-bit floating-point format E4M3 (1 sign bit, 4
 * exponent bits with bias 7, 3 mantissa bits, subnormals m/8 * 2^-6, no
 * infinities; 0x7f / 0xff are NaN and never written):
 *   kv_cache_layer  uint8 [2][num_blocks][16][num_kv_heads][head_dim] codes,
 *   kv_scales       float32 [2][num_blocks][num_kv_heads][16] scales (as INT8),
 * value = E4M3(code) * scale, with scale = max|x| / 448 and code = the E4M3
 * value nearest to x / scale (IEEE float32 quotient, magnitude clipped at
 * 448), ties to the even code, sign bit from the quotient; an all-zero row
 * has scale 0 and codes 0.
 *
 * paged_kv_write_fp8 — quantise and store the step's new K/V, as
 *   paged_kv_write_int8.
 * paged_attention_fp8 — paged_attention over such a cache, with the kernels
 *   of paged_attention_int8: the codes become bf16 (exact) or float32 before
 *   the products and the scales enter as for INT8.
 * Arguments, workspace and error conventions are those of the INT8 calls.
 */
int paged_kv_write_fp8(const void* k, const void* v, const int64_t* slot_mapping, void* kv_cache_layer,
                       float* kv_scales, int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                       int32_t head_dim, int32_t dtype, int32_t* device_error, void* stream);
int paged_attention_fp8(void* out, const void* q, const void* kv_cache_layer, const float* kv_scales,
                        const int32_t* block_table, const int32_t* seq_lens,
                        const int32_t* query_start_loc, const int32_t* num_computed_tokens,
                        float scale, int32_t num_reqs, int64_t num_tokens, int32_t num_q_heads,
                        int32_t num_kv_heads, int32_t head_dim, int32_t num_blocks,
                        int32_t max_blocks_per_req, int32_t max_query_len, int32_t max_seq_len,
                        int32_t dtype, void* workspace, size_t workspace_bytes, void* stream,
                        void* const* phase_events);

/*
 * paged_kv_copy_blocks — copy whole cache blocks (K and V, every kv head):
 * the copy half of copy-on-write prefix sharing (lpnh.cn/news/2436702,
 * section 2.2: sequences share prefix blocks and a block is copied only
 * when they diverge inside it).
 *
 *   kv_cache_layer  device, [2][num_blocks][16][num_kv_heads][head_dim], dtype.
 *   copies          device int32 [num_copies][2]: (source block, destination
 *                   block).  No block may be the destination of two pairs or
 *                   both a source and a destination (the order of the copies
 *                   is unspecified).  A pair with an id outside
 *                   [0, num_blocks) is skipped and sets PKV_DEVERR_BLOCK_ID.
 *   device_error    device int32, or NULL.
 *   num_copies      >= 0 (0 enqueues nothing).
 * The destination gets the source's bits.  Returns PKV_OK or an argument
 * error; enqueued on `stream`.
 */
int paged_kv_copy_blocks(void* kv_cache_layer, const int32_t* copies, int32_t num_copies,
                         int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                         int32_t* device_error, void* stream);

/*
 * Host block manager and step scheduler (no HIP call, no device memory):
 * builds each step's metadata for paged_kv_write / paged_attention.
 *
 * The cache is a pool of num_blocks 16-token blocks allocated up front; a
 * request's block table grows by the next free block when its last block is
 * full, and its blocks return to the pool when it finishes
 * (lpnh.cn/news/2436702, section 2.2; "大模型推理部署：从单卡到集群的工程化落地
 * 路径", section 2.2).  Requests may share prefix blocks; a shared block is
 * copied before a step writes into it (copy-on-write).  Each step schedules,
 * per request, the tokens between num_computed_tokens and num_tokens, with
 * no prefill / decode distinction, under four limits: max_num_seqs, the
 * token budget, max_model_len and the free blocks ("AI Infra入门干货总结",
 * section "连续批处理").
 *
 * Policy where the pages are silent: first come, first served; a request
 * that cannot get a block this step is skipped (it waits; no preemption) and
 * later requests may still run; a request gets as many pending tokens as the
 * limits allow (a partial chunk is a chunked prefill); free blocks are
 * handed out first in, first out (initially 0, 1, 2, ...; freed blocks join
 * the back in table order); a copy-on-write takes its free block before the
 * request's new blocks; unused block-table entries are -1.
 *
 * Use: add / fork / append / finish requests, then pkv_bm_schedule fills a
 * pkv_step; the caller copies its arrays to the device, runs
 * paged_kv_copy_blocks(step.copies) and paged_kv_write(slot_mapping) before
 * paged_attention, then calls pkv_bm_commit.  Nothing else may change the
 * manager between schedule and commit.  A manager is not thread-safe.
 * Every call returns a pkv_status (PKV_ERR_METADATA for an unknown or
 * duplicate request id or a call out of order; pkv_last_error_detail()
 * says which).
 */
typedef struct pkv_block_manager pkv_block_manager;

typedef struct {
  /* limits of the step, set by the caller */
  int32_t max_num_seqs;   /* requests per step, > 0 */
  int32_t token_budget;   /* tokens per step, > 0 */
  int32_t max_model_len;  /* tokens per request, > 0 */
  /* HOST output arrays owned by the caller */
  int64_t* req_ids;              /* [max_num_seqs] request id of each row */
  int32_t* query_start_loc;      /* [max_num_seqs + 1] */
  int32_t* seq_lens;             /* [max_num_seqs] */
  int32_t* num_computed_tokens;  /* [max_num_seqs] */
  int32_t* block_table;          /* [max_num_seqs][max_blocks_per_req], -1 = unused */
  int64_t* slot_mapping;         /* [token_budget] */
  int32_t* copies;               /* [max_num_seqs][2] (source, destination) blocks */
  /* results */
  int32_t num_reqs, num_tokens, num_copies, max_query_len, max_seq_len;
} pkv_step;

/* A manager of num_blocks blocks; block tables have max_blocks_per_req
 * columns.  *out receives the handle (free it with pkv_bm_destroy). */
int pkv_bm_create(int32_t num_blocks, int32_t max_blocks_per_req, pkv_block_manager** out);
void pkv_bm_destroy(pkv_block_manager* bm);
/* A new request of num_prompt_tokens (>= 1) pending tokens. */
int pkv_bm_add_request(pkv_block_manager* bm, int64_t req_id, int32_t num_prompt_tokens);
/* The same, sharing the first min(prefix_tokens, computed tokens of
 * prefix_from, num_prompt_tokens - 1) / 16 full blocks of request
 * prefix_from, which count as computed (a prefix-cache hit).  The caller
 * guarantees that those tokens are the same. */
int pkv_bm_add_request_with_prefix(pkv_block_manager* bm, int64_t req_id, int32_t num_prompt_tokens,
                                   int64_t prefix_from, int32_t prefix_tokens);
/* child_id continues from parent_id's state, sharing all of its blocks. */
int pkv_bm_fork(pkv_block_manager* bm, int64_t parent_id, int64_t child_id);
/* n >= 0 more tokens (e.g. a sampled token) for the request. */
int pkv_bm_append_tokens(pkv_block_manager* bm, int64_t req_id, int32_t n);
/* The request leaves; blocks no other request shares return to the pool. */
int pkv_bm_finish(pkv_block_manager* bm, int64_t req_id);
/* Free blocks (-1 for a NULL manager). */
int32_t pkv_bm_num_free_blocks(const pkv_block_manager* bm);
/* A request's num_tokens, num_computed_tokens and block count; its first
 * min(max_blocks, count) block ids go to `blocks` (HOST, may be NULL). */
int pkv_bm_request_state(const pkv_block_manager* bm, int64_t req_id, int32_t* num_tokens,
                         int32_t* num_computed, int32_t* blocks, int32_t max_blocks, int32_t* num_blocks);
/* Schedule one step into *step (see pkv_step); allocates blocks and records
 * the step's copy-on-write pairs. */
int pkv_bm_schedule(pkv_block_manager* bm, pkv_step* step);
/* The scheduled step ran: its tokens count as computed. */
int pkv_bm_commit(pkv_block_manager* bm);

/* Static text of a pkv_status. */
const char* pkv_status_string(int status);

/* Detail of the last error returned on the calling thread ("" if none). */
const char* pkv_last_error_detail(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_KV_H_ */
