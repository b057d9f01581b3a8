/*
 * pic.h -- C ABI of the position-free paged attention library (libpic.so).
 *
 * The operation is the one of "MiniPIC: Flexible Position-Independent Caching
 * in <100LOC", §2.1 (Position-free KV implementation): keys are cached
 * UNROTATED in fixed-size physical blocks that several requests may share at
 * different logical offsets, and the attention kernel applies the rotary
 * rotation on the fly from a cosine/sine table indexed by each request's own
 * logical positions:
 *
 *     score(t, j) = (R_t q_t)^T (R_pi(j) k~_j) / sqrt(d)
 *
 * with pi(j) the logical position of stored key j in the current request.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pointers: every array argument is DEVICE memory owned by the caller,
 *   unless the argument is documented as host memory.  The library never
 *   allocates or frees device memory and keeps no state between calls; the
 *   exceptions are the host-side scheduler object of pic_sched_* (plain
 *   host memory, created and destroyed by the caller's calls) and the
 *   per-thread measurement events of pic_set_kernel_events.
 * - stream: a hipStream_t (NULL = the legacy default stream).  Every call
 *   only enqueues work on that stream and returns without synchronising the
 *   host.
 * - Return value: PIC_OK (0) or a negative pic_status.  Problems that can be
 *   seen on the host (null pointers, unsupported shapes or dtypes, a
 *   workspace that is too small) are reported before anything is launched.
 *   PIC_EHIP means a HIP launch reported an error.
 * - Device-resident values are PRECONDITIONS (checked by
 *   pic_validate_metadata on host copies, not by the kernels): block ids in
 *   [0, num_blocks), positions in [0, max_pos), 1 <= q_len <= seq_len,
 *   seq_len <= max_seq_len, cu_seqlens consistent.  The kernels clamp block
 *   ids and positions into range so that a violated precondition yields wrong
 *   numbers, never an out-of-bounds access.
 * - Supported shapes: head_dim in {64, 128}; block_size == 16;
 *   num_q_heads % num_kv_heads == 0 with group size Hq/Hkv in {1,2,4,8,16}.
 *
 * Memory layouts (row-major, element type = dtype)
 * ------------------------------------------------
 *   k_pool  [num_blocks][Hkv][block_size][head_dim]   unrotated keys
 *   v_pool  [num_blocks][Hkv][head_dim][block_size]   values, transposed per block
 *   cache slot s = block * block_size + offset.
 *   q, out  [rows][Hq][head_dim]  (one row per query token)
 *   cos_tab, sin_tab  float32 [max_pos][head_dim/2]
 *
 * Readings of the page that the ABI fixes (the page is silent on them):
 *   rotate-half pairing (element i with i + d/2); theta_i = base^(-2i/d);
 *   q head h reads kv head h / (Hq/Hkv); V is not rotated; query row i of a
 *   request with q_len rows and seq_len slots sees slots j <= seq_len - q_len
 *   + i (causal, bottom-right aligned, over slot index -- positions never
 *   affect the mask); softmax with the natural exponential.
 */
#ifndef PIC_H_
#define PIC_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    PIC_OK = 0,
    PIC_EINVAL = -1,        /* bad argument (null pointer, negative size, ...) */
    PIC_EUNSUPPORTED = -2,  /* shape or dtype outside the supported set */
    PIC_EWORKSPACE = -3,    /* workspace missing or smaller than required */
    PIC_EHIP = -4           /* a HIP call or kernel launch failed */
} pic_status;

typedef enum {
    PIC_F32 = 0,            /* float32 q, K, V, out */
    PIC_BF16 = 1            /* bfloat16 q, K, V, out (fp32 accumulation) */
} pic_dtype;

/* Human-readable name of a pic_status value.  Never returns NULL. */
const char* pic_status_string(int status);

/* Library version, as major * 10000 + minor * 100 + patch. */
int pic_version(void);

/*
 * pic_rope_table -- fill the cosine/sine lookup table (MiniPIC §2.1,
 * Implementation bullet: the kernel looks up a cosine/sine table for every
 * key element).
 *   cos_tab[p][i] = cos(p * theta_i), sin_tab[p][i] = sin(p * theta_i),
 *   theta_i = base^(-2i/head_dim), p in [0, max_pos), i in [0, head_dim/2).
 * Angles and trig are evaluated in float64 and stored as float32 (round to
 * nearest even).  Both outputs are float32 [max_pos][head_dim/2], device.
 * Errors: PIC_EINVAL for null outputs, max_pos <= 0, base <= 0;
 * PIC_EUNSUPPORTED for odd or non-positive head_dim.
 */
int pic_rope_table(float* cos_tab, float* sin_tab, int max_pos, int head_dim, double base,
                   void* stream);

/*
 * pic_cache_write -- store the step's new keys and values, UNROTATED, into
 * the paged pools (MiniPIC §2.1: the cache holds non-rotated key vectors, so
 * a block never has to be rewritten when it is reused at another offset).
 *   k, v          [num_tokens][Hkv][head_dim] (dtype), device, read only
 *   slot_mapping  int32 [num_tokens], device: cache slot of each token;
 *                 slots < 0 or >= num_blocks * block_size are skipped
 *   k_pool/v_pool the pools in the layouts above (written in place)
 * Bytes are copied unchanged (no arithmetic).  Two tokens mapped to the same
 * slot in one call race.  num_tokens == 0 is a no-op.
 * Errors: PIC_EINVAL (null pointers with num_tokens > 0, negative sizes),
 * PIC_EUNSUPPORTED (dtype, head_dim, block_size).
 */
int pic_cache_write(const void* k, const void* v, const int32_t* slot_mapping, int num_tokens,
                    int num_kv_heads, int head_dim, int dtype, void* k_pool, void* v_pool,
                    int num_blocks, int block_size, void* stream);

/*
 * pic_attn_workspace_size -- bytes of device workspace that pic_attn_decode /
 * pic_attn_prefill need for these bounds (total_q = number of query rows,
 * max_seq_len >= every seq_len).  It holds the work list of the mixed
 * launch and the per-chunk partial results of split requests and split
 * prefill tiles; every call
 * writes what it reads, so it needs no initialisation and can be reused by
 * later calls on the same stream.  Calls that overlap in time must use
 * different workspaces.
 * Returns 0 for unsupported arguments.
 */
size_t pic_attn_workspace_size(int num_reqs, int total_q, int max_seq_len, int num_q_heads,
                               int num_kv_heads, int head_dim, int dtype);

/*
 * pic_attn_decode -- one query row per request (q_len == 1), the
 * memory-bound path.  Request r's query is row r of q; it sits at logical
 * position q_pos[r] and attends to key slots 0..seq_lens[r]-1, whose logical
 * positions are k_pos[cu_seqlens_k[r] + j] (= pi(j), MiniPIC §2.1 score
 * equation).  Slot j of request r lives in physical block
 * block_table[r * block_table_stride + j / block_size] at offset
 * j % block_size.  Long contexts are split into chunks whose count depends
 * only on seq_len (so a request's result does not depend on the rest of the
 * batch); a second small kernel on the same stream merges the chunks'
 * partial results.
 *   q        [num_reqs][Hq][head_dim] unrotated, dtype
 *   q_pos    int32 [num_reqs]
 *   out      [num_reqs][Hq][head_dim], dtype (written)
 *   workspace  >= pic_attn_workspace_size(num_reqs, num_reqs, max_seq_len, ...)
 * A request with seq_len == 0 gets a zero output row.  The pools, tables and
 * metadata are only read.
 */
int pic_attn_decode(const void* q, const int32_t* q_pos, const void* k_pool, const void* v_pool,
                    const int32_t* block_table, int block_table_stride, const int32_t* seq_lens,
                    const int32_t* cu_seqlens_k, const int32_t* k_pos, const float* cos_tab,
                    const float* sin_tab, int max_pos, int num_reqs, int num_q_heads,
                    int num_kv_heads, int head_dim, int block_size, int num_blocks,
                    int max_seq_len, int dtype, void* out, void* workspace,
                    size_t workspace_bytes, void* stream);


/*
 * pic_attn_decode_append -- pic_attn_decode that also writes the step's new
 * tokens (MiniPIC §2.1: the cache holds keys unrotated; the write itself is
 * pic_cache_write's).  Request r's new token is its key slot
 * seq_lens[r] - 1: new_k and new_v [num_reqs][Hkv][head_dim] (dtype; row r =
 * request r) are stored, unrotated, at offset (seq_lens[r] - 1) % block_size
 * of block block_table[r * block_table_stride + (seq_lens[r] - 1) /
 * block_size], and the same call attends to them there.  The pools then hold
 * the same bytes, and out the same values bit for bit, as pic_cache_write of
 * those rows followed by pic_attn_decode.  The work of the write is done by
 * the decode launch itself (each request's last key chunk stores its token
 * and uses it for its own key slot), which saves the separate write launch
 * of a decode step.  Preconditions beyond pic_attn_decode's: seq_lens[r] >= 1,
 * and no other request of the call reads the slot being written (a decode
 * appends to its own tail block).  A request with seq_len == 0 writes
 * nothing.  A block id out of range is not written (the attention reads it
 * clamped, as everywhere).  Errors as pic_attn_decode; PIC_EINVAL when
 * new_k or new_v is NULL.  The pools are written; the rest is only read.
 */
int pic_attn_decode_append(const void* q, const void* new_k, const void* new_v,
                           const int32_t* q_pos, const void* k_pool, const void* v_pool,
                           const int32_t* block_table, int block_table_stride,
                           const int32_t* seq_lens, const int32_t* cu_seqlens_k,
                           const int32_t* k_pos, const float* cos_tab, const float* sin_tab,
                           int max_pos, int num_reqs, int num_q_heads, int num_kv_heads,
                           int head_dim, int block_size, int num_blocks, int max_seq_len,
                           int dtype, void* out, void* workspace, size_t workspace_bytes,
                           void* stream);
/*
 * pic_attn_decode_noalloc -- pic_attn_decode for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same kernels and the same results,
 * bit for bit, with no workspace argument.  The chunk partials go to a
 * fixed array of 64 MiB that the library holds on each device it runs on
 * until the process ends (its address is looked up once per device, on the
 * first call with that device current: make that first call outside HIP graph
 * capture; later calls can be captured).  The call itself allocates nothing.
 * The array needs no initialisation (every call writes what it reads) and
 * keeps the last call's contents; calls that overlap in time on one device
 * race on it, so the caller serialises them (one stream, or events).
 * Arguments, layouts and preconditions as in pic_attn_decode.
 * Errors as pic_attn_decode, plus PIC_EWORKSPACE when the batch needs more
 * than the 64 MiB, i.e. when pic_attn_workspace_size(num_reqs, num_reqs,
 * max_seq_len, ...) without its prefill-split part exceeds 67,108,864 bytes
 * (for the 32 / 8 heads, d = 128 layer: about 2 million keys over the whole
 * batch; 64 x 4,097 keys use 8.5 MB, 4 x 131,073 keys 17.1 MB), and
 * PIC_EHIP when the array's device address cannot be obtained.
 */
int pic_attn_decode_noalloc(const void* q, const int32_t* q_pos, const void* k_pool,
                            const void* v_pool, const int32_t* block_table,
                            int block_table_stride, const int32_t* seq_lens,
                            const int32_t* cu_seqlens_k, const int32_t* k_pos,
                            const float* cos_tab, const float* sin_tab, int max_pos,
                            int num_reqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_seq_len, int dtype,
                            void* out, void* stream);

/*
 * pic_attn_decode_shared -- pic_attn_decode with the key chunks of each
 * request cut where its blocks say, so that blocks shared by several requests
 * are read once per XCD instead of once per request (MiniPIC §2.1: one
 * physical block serves concurrent requests at different offsets).  A block
 * whose physical id hashes to a fixed residue (probability 1/16) starts a new
 * chunk unless another such block lies among the 11 blocks before it; a gap
 * of more than 38 blocks between two cuts is cut into equal parts of at most
 * 24 blocks.  Two requests holding the
 * same span at different offsets therefore cut it at the same blocks, and a
 * planner groups chunks by their first physical block so that identical
 * chunks run side by side on one XCD and the later ones find the span in
 * that XCD's L2.  The chunking depends only on the request's own block table,
 * so a request's output does not depend on the rest of the batch; it differs
 * from pic_attn_decode's by floating-point rounding only.  Arguments,
 * layouts and preconditions as in pic_attn_decode, except the workspace:
 *   workspace >= pic_attn_decode_shared_workspace_size(num_reqs, max_seq_len,
 *                                                      Hq, Hkv, head_dim, dtype)
 * PIC_EUNSUPPORTED when a context spans more than 65536 blocks (1,048,576
 * keys).  Three small launches (chunking, ordering, merge) surround the
 * decode kernel.
 */
int pic_attn_decode_shared(const void* q, const int32_t* q_pos, const void* k_pool,
                           const void* v_pool, const int32_t* block_table,
                           int block_table_stride, const int32_t* seq_lens,
                           const int32_t* cu_seqlens_k, const int32_t* k_pos,
                           const float* cos_tab, const float* sin_tab, int max_pos,
                           int num_reqs, int num_q_heads, int num_kv_heads, int head_dim,
                           int block_size, int num_blocks, int max_seq_len, int dtype,
                           void* out, void* workspace, size_t workspace_bytes, void* stream);
/* Bytes of workspace pic_attn_decode_shared needs; 0 for unsupported shapes
 * or dtypes, or a max_seq_len beyond 65536 blocks. */
size_t pic_attn_decode_shared_workspace_size(int num_reqs, int max_seq_len, int num_q_heads,
                                             int num_kv_heads, int head_dim, int dtype);

/*
 * pic_attn_prefill -- any mix of requests in ONE launch (chunked prefill,
 * span prefill, and q_len == 1 decodes side by side: the interleaved
 * span-prefill schedule of MiniPIC §2.2 "Scheduling" puts span prefills and
 * ongoing decodes in the same batch).  Request r owns query rows
 * cu_seqlens_q[r] .. cu_seqlens_q[r+1]-1 of q; query row i of the request
 * (0-based) sits at position q_pos[cu_seqlens_q[r] + i] and sees key slots
 * j <= seq_lens[r] - q_len + i.  max_q_len must be >= every q_len (a
 * precondition, like the others; no kernel reads it).  Other arguments as in
 * pic_attn_decode.  A small planner kernel builds the work list in the
 * workspace first.  If the device metadata break a precondition so that the
 * work list would not fit the workspace (for instance cu_seqlens_q not
 * ascending, so that requests' rows overlap), the planner runs nothing and
 * every output row of the launch (as cu_seqlens_q delimits them, clipped to
 * [0, total_q)) is filled with NaN; the call still returns PIC_OK, since the
 * host never reads device data.
 * bf16 launches with fewer prefill tiles (256 query rows of one kv head)
 * than 256 split each tile over a context of 2048 keys or more into key
 * chunks that run in parallel; a merge kernel on the same stream combines
 * them.  The split depends on the whole launch, so a request's prefill rows
 * are bit-identical between launches that split it the same way (always
 * when both launches have 256 tiles or more) and otherwise agree within
 * rounding.
 *   q, out   [total_q][Hq][head_dim]
 *   workspace >= pic_attn_workspace_size(num_reqs, total_q, max_seq_len, ...)
 */
int pic_attn_prefill(const void* q, const int32_t* cu_seqlens_q, const int32_t* q_pos,
                     const void* k_pool, const void* v_pool, const int32_t* block_table,
                     int block_table_stride, const int32_t* seq_lens,
                     const int32_t* cu_seqlens_k, const int32_t* k_pos, const float* cos_tab,
                     const float* sin_tab, int max_pos, int num_reqs, int total_q,
                     int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int num_blocks, int max_seq_len, int dtype, void* out,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * In-kernel-rotation ablation: the conventional RoPE cache that the
 * position-free design replaces, and the same attention kernels with the key
 * rotation compiled out.  MiniPIC §2.1 (Implementation) moves the rotation of
 * keys from the cache write into the attention kernel at the price of a
 * table lookup and a few fused multiply-adds per key element; the page puts
 * that price at 5.7 % of end-to-end time (§4).  These entry points measure
 * it at kernel level on MI355X: same shapes, same kernels, keys pre-rotated.
 *
 * pic_cache_write_rotated -- like pic_cache_write, but each key is rotated
 * to positions[t] (int32 [num_tokens], device) before it is stored:
 *   k_pool slot = round(R_p k~)  (rotate-half, fp32 arithmetic with the
 *   table's float32 cos/sin, rounded to dtype);  V is copied unchanged.
 * A block written this way is valid at that one offset only (it cannot be
 * shared at another offset, which is the point of the comparison).
 * cos_tab/sin_tab: float32 [max_pos][head_dim/2] from pic_rope_table;
 * positions are clamped into [0, max_pos).  Errors as pic_cache_write, plus
 * PIC_EINVAL for null positions/tables or max_pos <= 0.
 */
int pic_cache_write_rotated(const void* k, const void* v, const int32_t* slot_mapping,
                            const int32_t* positions, const float* cos_tab,
                            const float* sin_tab, int max_pos, int num_tokens,
                            int num_kv_heads, int head_dim, int dtype, void* k_pool,
                            void* v_pool, int num_blocks, int block_size, void* stream);

/*
 * pic_attn_decode_rotated / pic_attn_prefill_rotated -- pic_attn_decode /
 * pic_attn_prefill for a k_pool that already holds every key rotated to the
 * position at which this request uses it (for instance written by
 * pic_cache_write_rotated).  The kernels are the position-free ones with the
 * key-side table lookup and rotation removed; there is no cu_seqlens_k /
 * k_pos argument.  The query is still rotated in the kernel by q_pos, with
 * cos_tab/sin_tab.  All other arguments, layouts and the workspace are as in
 * the position-free calls.  dtype must be PIC_BF16 (else PIC_EUNSUPPORTED).
 */
int pic_attn_decode_rotated(const void* q, const int32_t* q_pos, const void* k_pool,
                            const void* v_pool, const int32_t* block_table,
                            int block_table_stride, const int32_t* seq_lens,
                            const float* cos_tab, const float* sin_tab, int max_pos,
                            int num_reqs, int num_q_heads, int num_kv_heads, int head_dim,
                            int block_size, int num_blocks, int max_seq_len, int dtype,
                            void* out, void* workspace, size_t workspace_bytes, void* stream);
int pic_attn_prefill_rotated(const void* q, const int32_t* cu_seqlens_q, const int32_t* q_pos,
                             const void* k_pool, const void* v_pool,
                             const int32_t* block_table, int block_table_stride,
                             const int32_t* seq_lens, const float* cos_tab,
                             const float* sin_tab, int max_pos, int num_reqs, int total_q,
                             int max_q_len, int num_q_heads, int num_kv_heads, int head_dim,
                             int block_size, int num_blocks, int max_seq_len, int dtype,
                             void* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * pic_blocks_copy -- copy whole KV blocks between two pools: block
 * src_blocks[i] of (src_k_pool, src_v_pool) goes to block dst_blocks[i] of
 * (dst_k_pool, dst_v_pool), K and V, bytes unchanged.  For CPU offload of
 * position-free blocks (MiniPIC §3, "native compatibility": unrotated
 * blocks move between GPU and host without tracking or adjusting positions):
 * either pool may be device memory or PINNED host memory allocated with
 * hipHostMalloc (torch: pin_memory=True), which the kernel reads or writes
 * over the host link.  Both pools use the layouts above with the same
 * num_kv_heads, head_dim and dtype; src_blocks/dst_blocks are int32
 * [num_pairs] in device-accessible memory (device or pinned host).  A pair
 * with an id outside [0, num_src_blocks) or [0, num_dst_blocks) is skipped.
 * Pairs writing the same destination block race.  Stream-ordered like
 * every other call: synchronise the stream before the host reads a host
 * pool.  Errors: PIC_EINVAL (negative sizes, null pointers with
 * num_pairs > 0), PIC_EUNSUPPORTED (dtype, head_dim, block_size).
 */
int pic_blocks_copy(const void* src_k_pool, const void* src_v_pool, const int32_t* src_blocks,
                    int num_src_blocks, void* dst_k_pool, void* dst_v_pool,
                    const int32_t* dst_blocks, int num_dst_blocks, int num_pairs,
                    int num_kv_heads, int head_dim, int dtype, int block_size, void* stream);

/*
 * Span-aware block hashing (host code, no device work).  MiniPIC §2.2
 * ("user-controlled cache reuse primitives"): spans are padded to KV-block
 * boundaries, and two special tokens at the START of a block change how that
 * block's prefix-cache hash is chained, which decides which blocks requests
 * share:
 *   default            h_i = H(h_{i-1}, x_i)
 *   SSEP at block start h_i = H(h_0, x_i)       chain restarts: the span is
 *                                               cacheable whatever precedes it
 *   PDEP at block start h_i = H(h_0, x_{<=i})   depends on the whole prompt up
 *                                               to block i (no false hits)
 * x_i = token ids of block i, h_0 = seed, h_{-1} = h_0.  H is FNV-1a 64 over
 * the little-endian bytes of the 8-byte parent hash followed by each token as
 * 4 bytes (for PDEP: h_0 followed by every token of blocks 0..i).  A special
 * token anywhere else is an ordinary token.  Pass -1 to disable a primitive.
 * Only full blocks are hashed; a trailing partial block is never shared.
 *
 * pic_block_hashes -- hashes of the full blocks of one token sequence.
 *   tokens  int32 [num_tokens], HOST;  hashes  uint64 [num_tokens / block_size], HOST
 * Returns the number of hashes written (>= 0), or PIC_EINVAL (num_tokens < 0,
 * block_size <= 0, null pointers with at least one full block).
 */
int pic_block_hashes(const int32_t* tokens, int num_tokens, int block_size, int32_t ssep_token,
                     int32_t pdep_token, uint64_t seed, uint64_t* hashes);

/*
 * pic_build_block_tables -- the attention metadata of a batch of prompts with
 * block sharing decided by the hashes above (all arrays HOST memory).
 *   tokens      int32 [cu_seqlens[num_reqs]]: the prompts, concatenated
 *   cu_seqlens  int32 [num_reqs + 1], cu_seqlens[0] == 0
 *   block_size  must be 16 (the attention kernels' block size)
 *   first_block, num_blocks: new physical blocks are numbered first_block,
 *               first_block + 1, ... and must stay below num_blocks
 * Outputs:
 *   block_table  int32 [num_reqs][block_table_stride] (unused entries 0):
 *                full blocks with equal hashes (across and within requests)
 *                map to one physical block, numbered in order of first use;
 *                a partial last block always gets its own block
 *   k_pos        int32 [total tokens]: pi(j) = j, the token's index in its
 *                request (positions run over the composed prompt)
 *   slot_mapping int32 [total tokens]: the cache slot to write each token's
 *                K/V to (pic_cache_write), or -1 where an earlier occurrence of
 *                the same block in the batch writes it
 *   block_hashes uint64 [sum of full blocks], may be NULL
 *   num_new_blocks  physical blocks used
 * Returns PIC_OK, or PIC_EINVAL for bad sizes, a table too narrow for a
 * request, or a pool too small (num_blocks reached).
 */
int pic_build_block_tables(const int32_t* tokens, const int32_t* cu_seqlens, int num_reqs,
                           int block_size, int32_t ssep_token, int32_t pdep_token,
                           uint64_t seed, int first_block, int num_blocks,
                           int32_t* block_table, int block_table_stride, int32_t* k_pos,
                           int32_t* slot_mapping, uint64_t* block_hashes,
                           int* num_new_blocks);

/*
 * pic_validate_metadata -- check the device-value preconditions above on
 * HOST copies of the metadata (test and debug helper; no device work).
 * cu_seqlens_q may be NULL for a decode batch (one query per request).
 * Returns PIC_OK or PIC_EINVAL; when msg is not NULL a description of the
 * first violation is written into msg[0..msg_len-1] (NUL terminated).
 */
int pic_validate_metadata(const int32_t* cu_seqlens_q, const int32_t* q_pos,
                          const int32_t* block_table, int block_table_stride,
                          const int32_t* seq_lens, const int32_t* cu_seqlens_k,
                          const int32_t* k_pos, int num_reqs, int total_q, int max_seq_len,
                          int max_pos, int num_blocks, int block_size, char* msg, int msg_len);

/*
 * pic_decode_num_splits -- number of key chunks S a q_len == 1 request with
 * seq_len keys is split into by the attention kernels: round(seq_len / 512),
 * at least 1, at most one per inner step of 32 (bf16) or 16 (fp32) keys.  A
 * pure function of seq_len and dtype, so a request's result does not depend
 * on its batch.  pic_decode_chunk_start gives the first key of chunk
 * 0 <= chunk <= S (chunk S starts at seq_len; -1 outside that range): the
 * inner steps are dealt out evenly, so chunks differ by at most one step.
 * pic_decode_split_len gives the key slots of the longest chunk (its inner
 * steps times 32 or 16).
 */
int pic_decode_num_splits(int seq_len, int dtype);
int pic_decode_chunk_start(int seq_len, int chunk, int dtype);
int pic_decode_split_len(int seq_len, int dtype);

/*
 * pic_set_kernel_events -- measurement hook.  While set (both non-null
 * hipEvent_t handles, passed as void*, created with timing enabled), every
 * attention call made from the calling host thread hands them to the
 * dispatch of its main kernel (decode_kernel for pic_attn_decode and
 * pic_attn_decode_rotated, decode_shared_kernel for pic_attn_decode_shared,
 * mixed_kernel for pic_attn_prefill*), which records `before` at the
 * kernel's start and `after` at its end (hipExtLaunchKernel's start and
 * stop events: no extra packets on the stream).  So
 * hipEventElapsedTime(before, after) is that kernel's duration alone,
 * without the planning and merge launches of the call.  The setting is per
 * host thread; both null turns it off.  The events stay owned by the
 * caller.  Errors: PIC_EINVAL when exactly one handle is null; an attention
 * call returns PIC_EHIP when the launch fails.
 */
int pic_set_kernel_events(void* before, void* after);

/*
 * pic_timing_event_create / _record / _elapsed_ms / _destroy -- measurement
 * helpers: HIP events (hipEvent_t, passed as void*) created without the
 * system-scope acquire / release fence of a default event
 * (hipEventDisableSystemFence).  A default event's record writes back and
 * invalidates caches and slows the work after it (on a 64-request decode step
 * about 5-9 us per step with the pair of pic_set_kernel_events set, against
 * about 2 us for these); nothing may read device memory through these events,
 * they only time.  _create records the new event once on the default stream
 * (so an unused pair reads 0 ms) and stores it in *event; _record records it
 * on `stream`; _elapsed_ms writes the time from `start` to `stop` (both
 * complete) in ms; _destroy frees it (NULL: no-op).  The library calls are
 * the ones of the HIP runtime the library itself uses.  Errors: PIC_EINVAL for
 * a NULL argument (except _destroy), PIC_EHIP when HIP reports an error.
 */
int pic_timing_event_create(void** event);
int pic_timing_event_record(void* event, void* stream);
int pic_timing_event_elapsed_ms(void* start, void* stop, float* ms);
int pic_timing_event_destroy(void* event);

/*
 * pic_stream_read -- measurement helper: read `bytes` of device memory at
 * `src` once, with 16-byte loads (`workgroups` workgroups of 256 lanes
 * striding over the buffer in 4 KiB segments, 8 segments per iteration), the
 * plain streaming-read rate that the memory-bound decode path is compared
 * with on the same device.  order: NULL reads the buffer front to back;
 * otherwise int32 [bytes / piece_bytes] (device) lists pieces of piece_bytes
 * (a multiple of 4096) to read whole in that order -- with a random
 * permutation this is how a paged cache's scattered blocks are read.  An
 * entry outside [0, bytes / piece_bytes) reads the last piece.  sink: device memory of
 * at least workgroups * 256 uint32, almost never written (a lane stores only
 * when its folded data equals a fixed constant; the stores keep the loads
 * alive).  Errors: PIC_EINVAL for null pointers, bytes == 0 or not a multiple
 * of 4096, piece_bytes not a positive multiple of 4096 dividing bytes (when
 * order is given), workgroups outside [1, 2^20].
 */
int pic_stream_read(const void* src, size_t bytes, const int32_t* order, int piece_bytes,
                    int workgroups, void* sink, void* stream);

/*
 * Interleaved span-prefill scheduling (host)
 * ------------------------------------------
 * MiniPIC §2 (the scheduling paragraph after §2.2, ISPS) and §3,
 * contribution 4.  A scheduler object turns a trace of requests into engine
 * steps; each step is ONE mixed batch for pic_cache_write + pic_attn_prefill.
 *   PIC_SCHED_ISPS     every step mixes, under the token budget: one decode
 *                      token of every decoding request, then final-prompt
 *                      chunks, then span-prefill chunks;
 *   PIC_SCHED_BARRIER  one kind per step: span prefills while any running
 *                      request still waits for a span, else final prompts,
 *                      else decodes (the barrier-separated baseline).
 * Work model (tokens): a span is shared by id, a whole number of blocks, and
 * prefilled once on its own (causal, positions 0..len-1, blocks reserved
 * while any running request lists it); a request attends to its spans in
 * the listed order, then its final prompt (causal), then output_len decode
 * tokens, one per step.  Slot j of a request's composed sequence (spans'
 * blocks, then private blocks) has logical position j.  Admission: first come
 * first served by (arrival step, id), at most max_running at once, all of a
 * request's blocks reserved on admission; resident spans no running request
 * lists are evicted (least recently used first) when an admission needs
 * their blocks.
 * The scheduler is plain host memory created by pic_sched_create and freed by
 * pic_sched_destroy (the one stateful object of the library); spans and
 * requests are added before the first pic_sched_step.  Not thread-safe.
 */
typedef struct pic_sched pic_sched;

enum { PIC_SCHED_ISPS = 0, PIC_SCHED_BARRIER = 1 };
enum { PIC_SEQ_SPAN = 0, PIC_SEQ_PROMPT = 1, PIC_SEQ_DECODE = 2 };

/*
 * One step's batch.  The caller sets the capacities and points the arrays at
 * HOST memory of at least that size; pic_sched_step fills them and the
 * result fields.  Sequence i of the batch (a span chunk, a final-prompt
 * chunk or a decode token) owns query rows cu_seqlens_q[i]..cu_seqlens_q[i+1]
 * and key slots 0..seq_lens[i]-1; its new tokens are the query rows (the
 * caller writes their K/V to slot_mapping before the attention call).
 */
typedef struct {
  /* capacities (set by the caller) */
  int max_seqs;             /* sequences per step (>= max_running + spans in flight) */
  int max_rows;             /* query rows per step (>= token_budget) */
  long long max_keys;       /* sum of seq_lens per step */
  int block_table_stride;   /* >= blocks of the longest composed sequence */
  /* host arrays (caller-allocated) */
  int32_t* cu_seqlens_q;    /* [max_seqs + 1] */
  int32_t* q_pos;           /* [max_rows]   logical position of each query row */
  int32_t* slot_mapping;    /* [max_rows]   cache slot of each query row's token */
  int32_t* seq_lens;        /* [max_seqs] */
  int32_t* cu_seqlens_k;    /* [max_seqs + 1] */
  int32_t* k_pos;           /* [max_keys]   pi(j) = j of every sequence */
  int32_t* block_table;     /* [max_seqs][block_table_stride], unused entries 0 */
  int32_t* seq_kind;        /* [max_seqs]   PIC_SEQ_* */
  int32_t* seq_id;          /* [max_seqs]   span id or request id */
  int32_t* q_begin;         /* [max_seqs]   slot index of the sequence's first query row */
  /* results (written by pic_sched_step) */
  long long step;           /* index of this step (steps with no work count too) */
  int num_seqs, total_q, max_q_len, max_seq_len;
  long long total_keys;
  int num_finished;         /* requests that finished with this step */
} pic_sched_batch;

/* token_budget: query rows per step; block_size must be 16.  PIC_EINVAL for
 * an unknown policy or non-positive sizes. */
int pic_sched_create(int policy, int token_budget, int max_running, int num_blocks,
                     int block_size, pic_sched** sched);
void pic_sched_destroy(pic_sched* sched);
/* Returns the new span's id (0, 1, ...) or PIC_EINVAL (length not a positive
 * multiple of the block size, or stepping has started). */
int pic_sched_add_span(pic_sched* sched, int length);
/* Returns the new request's id (0, 1, ...) or PIC_EINVAL (unknown span id,
 * negative sizes, no span and no prompt, more blocks than the whole pool,
 * or stepping has started).  The request may be scheduled from step
 * arrival_step on. */
int pic_sched_add_request(pic_sched* sched, long long arrival_step, const int32_t* span_ids,
                          int num_spans, int prompt_len, int output_len);
/* Builds the next step into *batch: returns 1 (a step; num_seqs == 0 when no
 * admitted work exists yet at this step), 0 when every request has
 * finished, or PIC_EINVAL (null or too small arrays; the scheduler's state is
 * then unchanged, so the call can be repeated with larger arrays). */
int pic_sched_step(pic_sched* sched, pic_sched_batch* batch);

#ifdef __cplusplus
}
#endif

#endif /* PIC_H_ */
