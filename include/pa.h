/*
 * pa.h -- C ABI of libpa.so: paged KV cache and single-query decode attention
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (sources are the pages this project follows):
 *   - A pool of equal-size blocks holds the K and V vectors of many requests;
 *     each request has a block table mapping its logical blocks to physical
 *     blocks anywhere in the pool; position t of a request lives at offset
 *     t % b of physical block table[t / b].  ("Inside vLLM and TGI: Paging,
 *     Versioned Schedulers and Operations", section "Block addresses and
 *     fragmentation arithmetic"; "vLLM and PagedAttention: Virtual Memory for
 *     LLM Serving", paragraph 3.)
 *   - Decode attention reads a request's K/V through its table: for query
 *     head h of sequence i, with G = Hq / Hkv and g = h / G,
 *       s_t = scale * <q[i][h], K_i[t][g]>,  w = softmax(s over t < L_i),
 *       out[i][h] = sum_t w_t V_i[t][g].
 *     (transcript paragraph 3: the attention kernel reads through the
 *     mapping; the pages do not write the formula -- this is ordinary scaled
 *     dot-product attention of one query.)
 *   - Growing a request writes its new token's K/V into the slot its table
 *     gives; a shared, partially filled last block is copied to a private
 *     block before a write (copy-on-write).  ("Inside vLLM and TGI", section
 *     "Exact CPU block manager and copy-on-write"; transcript paragraph 4.)
 *
 * Conventions shared by every entry point
 *   - Ownership: the caller owns every buffer.  The library allocates and
 *     frees nothing and keeps no state between calls (no handles; calls are
 *     thread-safe).  Pointers marked "device" are device memory of the
 *     current HIP device; pointers marked "host" are host memory.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Every call that takes a stream only enqueues work on it and
 *     returns; inputs must stay alive and unmodified until the stream has
 *     passed the call (the stream form of "a worker still holding a lease
 *     keeps its blocks", "Inside vLLM and TGI", section "Exact CPU block
 *     manager and copy-on-write", last paragraphs).
 *   - Errors: host-side argument checks run first; a failed check returns a
 *     status and enqueues NOTHING, so a failing call has no side effect
 *     (the pages' atomic-failure rule for admission and copy-on-write).  A
 *     HIP launch error is reported as PA_ERR_HIP.  No exception crosses the
 *     ABI.
 *   - Device-resident contents (tables, lengths, slots, pairs) are not read
 *     by the host.  Kernels never access memory outside the buffers they are
 *     given: a table entry outside [0, num_blocks) contributes no tokens, a
 *     slot outside the pool is skipped, a length larger than the table or the
 *     stated maximum is clipped.  Results for such inputs are unspecified;
 *     pa_validate_tables reports them (the pages ask for a debug check of
 *     tables, bounds and lengths before a kernel reads them: "Inside vLLM
 *     and TGI", same section, validation paragraph).
 *
 * Pool layout (the ABI of the cache; chosen for gfx950, see each kernel)
 *   Two separate pools, K and V, each num_blocks * Hkv tiles of
 *   block_size * head_dim elements; tile (blk, h) starts at element
 *   (blk * Hkv + h) * block_size * head_dim, so every (block, KV head) tile is
 *   one contiguous run: 4 KiB for 16 x 128 16-bit or 16 x 64 fp32 elements,
 *   2 KiB at block_size 8, 8 KiB at block_size 32.
 *   Inside a tile, with R = min(block_size, 16) and tokens split into
 *   sub-tiles of R consecutive offsets (sub-tile s = o / R, row r = o % R,
 *   each sub-tile R * head_dim contiguous elements, in order):
 *     K, 16-bit pools: element (o, d) of sub-tile s at
 *          s*R*head_dim + (d / 32) * R*32 + r*32 + d % 32   ("[d/32][R][32]");
 *     K, fp32 pools: element (o, d) at o * head_dim + d (token-major);
 *     V: element (o, d) at ((o / 4) * head_dim + d) * 4 + o % 4
 *        -- groups of 4 tokens interleaved per dim ("[b/4][d][4]").
 *   The decode kernel's matrix-core loads then read whole 128-byte lines
 *   (1 KiB contiguous per 16-bit K instruction), each lane receiving its
 *   operand directly (8 dims of one token of K; 4 consecutive tokens of one
 *   dim of V); a token write touches 4 lines of K and 8 lines of V for 128
 *   16-bit dims.
 *
 * FP8 pools (PA_FP8_E4M3: OCP E4M3 without infinities, max 448, all-ones
 * mantissa and exponent = NaN; one byte per element) store codes with
 * per-KV-head scales from the descriptor, in sub-tiles of R rows (as above)
 * laid out for whole-line loads with permuted dimensions (D = head_dim):
 *     K: byte (r, d) at s*R*D + (d / (D/4)) * R*D/4 + ((d % (D/4)) / 16) * R*16
 *          + r*16 + d % 16;
 *     V: byte (r, d) at s*R*D + (r / 4) * 4*D + ((d % (D/16)) / 4) * 256
 *          + (d / (D/16)) * 16 + (d % 4) * 4 + r % 4.  The FP8 cache exists and its
 * usability depends on device, backend and scales ("Inside vLLM and TGI",
 * section "Launch a pinned engine from already reviewed local artifacts");
 * format and scaling here are this library's choice.  Writing value x of
 * head g stores the E4M3 value nearest to the fp32 quotient x / scale_g (ties
 * to even), saturated to +-448; NaN stores 0x7F.  For FP8 pools the inputs
 * k_new, v_new and q are bf16 and out_dtype is PA_F32 or PA_BF16.
 *
 * Supported shapes: block_size 8, 16 or 32; head_dim 64 or 128; dtype f32, f16, bf16, fp8;
 * 1 <= num_q_heads / num_kv_heads <= 16 and num_q_heads % num_kv_heads == 0.
 */
#ifndef PA_H
#define PA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Every entry point is exported with default visibility. */
#define PA_API __attribute__((visibility("default")))

typedef int32_t pa_status;
enum {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, negative size, inconsistent shape */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not built: dtype, head_dim, block_size, group */
  PA_ERR_WORKSPACE = 3,    /* workspace missing or smaller than pa_decode_workspace_size */
  PA_ERR_HIP = 4           /* the HIP runtime reported an error for a launch */
};

typedef int32_t pa_dtype;
enum { PA_F32 = 0, PA_F16 = 1, PA_BF16 = 2, PA_FP8_E4M3 = 3 };

/* partition_size value asking the library to choose (see pa_decode_attention). */
#define PA_PARTITION_AUTO (-1)

/* Describes a K/V pool pair (layout above).  Passed by pointer, read only
 * during the call. */
typedef struct pa_pool_desc {
  int32_t num_blocks;    /* physical blocks in each pool, >= 1 */
  int32_t block_size;    /* tokens per block (b); 8, 16 or 32 */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim;      /* 64 or 128 */
  pa_dtype dtype;        /* element type of both pools */
  /* PA_FP8_E4M3 pools only (NULL otherwise): device float [Hkv] per-KV-head
   * scales; a stored K code c of head g stands for value(c) * k_scales[g]. */
  const float* k_scales;
  const float* v_scales;
} pa_pool_desc;

/* Human-readable name of a status; never NULL, static storage. */
PA_API const char* pa_status_string(pa_status s);

/* Library version as major * 10000 + minor * 100 + patch. */
PA_API int32_t pa_version(void);

/*
 * pa_slot_mapping -- address translation for new tokens.
 *   slots[t] = table[seq][p / b] * b + p % b, with seq = seq_ids[t], p = positions[t]
 * ("Inside vLLM and TGI", section "Block addresses and fragmentation
 * arithmetic": logical block t // b, offset t % b, physical table[t // b]).
 *   block_tables  device int32 [num_seqs][max_blocks_per_seq], row-major
 *   seq_ids       device int32 [n]: row of block_tables for token t
 *   positions     device int32 [n]: zero-based position of token t
 *   slots         device int32 [n] (output); -1 where seq_id is outside
 *                 [0, num_seqs), the position is negative or past the table
 *                 row, the table entry is negative, or the slot overflows int32
 * n == 0 enqueues nothing and returns PA_OK.
 */
PA_API pa_status pa_slot_mapping(const int32_t* block_tables, int32_t max_blocks_per_seq,
                          int32_t num_seqs, const int32_t* seq_ids, const int32_t* positions,
                          int32_t n, int32_t block_size, int32_t* slots, void* stream);

/*
 * pa_write_kv -- write new tokens' K and V into their pool slots
 * (the device side of growing a request: "Inside vLLM and TGI", section
 * "Exact CPU block manager and copy-on-write"; transcript paragraph 3).
 *   k_pool, v_pool   device, pool layout above (written)
 *   k_new, v_new     device, pool dtype; token t, KV head h, dim d at
 *                    element t * new_stride + h * head_dim + d
 *   new_stride       elements between consecutive tokens (>= Hkv * head_dim;
 *                    Hkv * head_dim when contiguous [n][Hkv][d])
 *   slot_mapping     device int32 [n]; slot s is offset s % b of block s / b;
 *                    a slot < 0 or >= num_blocks * b is skipped
 * Bytes are copied unchanged (no conversion).  Two tokens with the same slot
 * in one call: unspecified which one lands.
 */
PA_API pa_status pa_write_kv(const pa_pool_desc* pool, void* k_pool, void* v_pool, const void* k_new,
                      const void* v_new, int64_t new_stride, const int32_t* slot_mapping,
                      int32_t n, void* stream);

/*
 * pa_copy_blocks -- copy whole blocks, all KV heads, in both pools
 * (copy-on-write of a shared partial last block: "Inside vLLM and TGI",
 * section "Exact CPU block manager and copy-on-write"; transcript paragraph 4).
 *   block_pairs  device int32 [n_pairs][2] = {src, dst}; a pair with an id
 *                outside [0, num_blocks) is skipped
 * Every dst must be distinct and must not appear as any src in the same call
 * (otherwise the result is unspecified).  n_pairs == 0 enqueues nothing.
 */
PA_API pa_status pa_copy_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                         const int32_t* block_pairs, int32_t n_pairs, void* stream);

/*
 * pa_decode_workspace_size -- bytes of device workspace pa_decode_attention
 * needs for these arguments (0 when no split is made: partition_size == 0,
 * every sequence fits in one partition, or PA_PARTITION_AUTO keeps one
 * pass): one fp32 record per (sequence, KV head, partition), or per (KV
 * head, unit) for a planned split, of G*head_dim + 2*G floats rounded up to
 * 128 bytes, G = Hq/Hkv; a planned split adds two int32 per sequence.
 * Splitting a sequence's context is not on the pages: the split and its
 * combine are the ordinary rescaling of partial softmax sums.
 * `bytes` is host memory; num_q_heads must be a multiple of num_kv_heads.
 */
PA_API pa_status pa_decode_workspace_size(const pa_pool_desc* pool, int32_t num_seqs,
                                   int32_t num_q_heads, int32_t max_context_len,
                                   int32_t partition_size, size_t* bytes);

/*
 * pa_decode_attention -- single-query decode attention through block tables
 * (formula at the top of this file).
 *   k_pool, v_pool    device, pool layout above (read)
 *   q                 device [num_seqs][num_q_heads][head_dim], pool dtype
 *   out               device [num_seqs][num_q_heads][head_dim] of out_dtype
 *                     (PA_F32, or the pool dtype: rounded to nearest even);
 *                     must not alias q or the pools
 *   block_tables      device int32 [num_seqs][max_blocks_per_seq]; entries
 *                     past ceil(L_i / b) are never read
 *   context_lens      device int32 [num_seqs]: L_i = number of stored tokens
 *                     attended to (positions 0 .. L_i - 1); L_i == 0 gives a
 *                     zero output row
 *   scale             multiplier of q.k (e.g. 1/sqrt(head_dim))
 *   max_context_len   host upper bound of every L_i (sizes the grid); lengths
 *                     above it are clipped to it
 *   partition_size    0: each (sequence, KV head) is one work unit; > 0:
 *                     positions are split into consecutive partitions of
 *                     partition_size tokens (a multiple of block_size),
 *                     processed independently and combined by a second
 *                     kernel that rescales each partition's (max, sum,
 *                     weighted sum) to the global max; PA_PARTITION_AUTO:
 *                     0 when num_seqs * Hkv already covers the GPU's
 *                     resident workgroups (per compute unit of the current
 *                     device: 3, FP8 pools 4, fp32 pools with head_dim 128 2)
 *                     or max_context_len <= 512; else the split is planned on
 *                     the device from the lengths: a sequence of n 16-token
 *                     tiles (8-token for 8-token blocks of FP8 and fp32
 *                     pools) is split into ceil(n / u) near-equal ranges, u
 *                     the smallest tile count of at least 512 tokens for which
 *                     each KV head's ranges number at most resident / Hkv --
 *                     one round of near-equal work units
 *                     (pa_decode_workspace_size with the same arguments on the
 *                     same device gives the matching workspace)
 *   workspace         device, >= pa_decode_workspace_size bytes (may be NULL
 *                     when that size is 0), 16-byte aligned; holds the
 *                     partial records (and, for a planned split, two ints per
 *                     sequence) of this call until its kernels finish in
 *                     stream order: calls that may overlap need separate
 *                     workspaces; its contents need no initialisation
 * Accumulation is fp32 in every dtype; q.k products of f16/bf16 inputs are
 * exact in fp32.
 */
PA_API pa_status pa_decode_attention(const pa_pool_desc* pool, const void* k_pool, const void* v_pool,
                              const void* q, void* out, pa_dtype out_dtype,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t num_seqs,
                              int32_t num_q_heads, float scale, int32_t max_context_len,
                              int32_t partition_size, void* workspace, size_t workspace_bytes,
                              void* stream);

/*
 * pa_decode_step -- one decode iteration in one launch: for every sequence i
 * with L_i >= 1, write row i of k_new / v_new (its current token) to
 * position L_i - 1, i.e. slot table[i][(L_i-1)/b]*b + (L_i-1)%b, then
 * attend over positions 0 .. L_i - 1 exactly as pa_decode_attention does.
 * Same result as pa_slot_mapping + pa_write_kv + pa_decode_attention with
 * those positions (the growth step of "Inside vLLM and TGI", section "Exact
 * CPU block manager and copy-on-write", followed by the attention step of the
 * transcript, paragraph 3).  The last block must already be private to the
 * sequence (copy-on-write done).
 *   k_pool, v_pool   device, pool layout above (one slot per sequence written)
 *   k_new, v_new     device, pool dtype; sequence i, KV head h, dim d at
 *                    element i * new_stride + h * head_dim + d
 *   new_stride       elements between sequences (>= Hkv * head_dim, 16-byte
 *                    multiple)
 *   other arguments as pa_decode_attention.  A table entry outside the pool
 *   for the current token's block: nothing is written and that block
 *   contributes no tokens.
 */
PA_API pa_status pa_decode_step(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                                const void* k_new, const void* v_new, int64_t new_stride,
                                const void* q, void* out, pa_dtype out_dtype,
                                const int32_t* block_tables, int32_t max_blocks_per_seq,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_q_heads, float scale, int32_t max_context_len,
                                int32_t partition_size, void* workspace, size_t workspace_bytes,
                                void* stream);

/* Size of the per-GPU device scratch behind pa_decode_step_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * pa_decode_step_noalloc -- pa_decode_step for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc): the same arguments without the workspace, the same
 * results.  A split's partial records live in a device array of
 * PA_NOALLOC_SCRATCH_BYTES (64 MiB) inside the library, one per GPU, created
 * when the library is loaded on that GPU and kept until the process ends;
 * the call itself allocates nothing.
 *   Returns PA_ERR_WORKSPACE, enqueueing nothing, when the call's workspace
 *   (pa_decode_workspace_size with the same arguments) exceeds that size, and
 *   PA_ERR_HIP when the array's address cannot be looked up on the current
 *   device.
 *   Every call on one GPU in a process shares that GPU's array, which keeps
 *   the last call's contents: calls that may overlap on one GPU (several
 *   streams or host threads) race and give undefined results; serialise
 *   them, or use pa_decode_step with separate workspaces.
 */
PA_API pa_status pa_decode_step_noalloc(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                                        const void* k_new, const void* v_new, int64_t new_stride,
                                        const void* q, void* out, pa_dtype out_dtype,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        int32_t num_q_heads, float scale, int32_t max_context_len,
                                        int32_t partition_size, void* stream);

/*
 * pa_prefill_attention -- multi-token (prefill or chunked-prefill) attention
 * through the block tables.  Sequence i stores L_i tokens; its chunk is the
 * n_i newest of them, n_i = q_start[i+1] - q_start[i] (positions L_i - n_i ..
 * L_i - 1, their K/V already written, e.g. by pa_write_kv).  Chunk row t sits
 * at position p = L_i - n_i + t and attends causally to positions 0 .. p:
 *     out[q_start[i] + t][h] = sum_{k <= p} softmax_k(scale * q[..][h] . K_i[k][g]) V_i[k][g]
 * with g = h / G as in decode.  In prefill all prompt tokens are known at once
 * (transcript, paragraph 1); a long prompt is processed in chunks over the
 * cached earlier tokens ("Inside vLLM and TGI", sections "Read the vLLM0.11.0
 * scheduler" and "Observability and debugging runbook").  n_i = L_i is a
 * whole prompt; n_i = 1 is one decode query.
 *   q              device [T][Hq][head_dim], pool dtype, 16-byte aligned;
 *                  T = q_start[num_seqs]
 *   out            device [T][Hq][head_dim] of out_dtype (PA_F32 or the pool
 *                  dtype), 16-byte aligned
 *   q_start        device int32 [num_seqs + 1], non-decreasing, q_start[0] = 0
 *   max_chunk_len  >= every n_i (host value; sizes the grid).  Rows of a
 *                  chunk past it are not computed.
 *   other arguments as pa_decode_attention (lengths clipped the same way).
 * A table entry outside the pool contributes no tokens: its block drops out
 * of every row's softmax and the other positions keep their places.
 * A row with p < 0 (n_i > L_i) gets zeros.  Accumulation is fp32.  For the
 * P.V products, bf16 and FP8 pools split P into high and low bf16 parts as in
 * decode (fp32-level results); fp16 pools round P to fp16 once (relative
 * 2^-11: about 5e-4 max row error on N(0,1) data, inside the 2e-3 bar).  A
 * 16-bit out_dtype is the rounding of the fp32 result.
 */
PA_API pa_status pa_prefill_attention(const pa_pool_desc* pool, const void* k_pool,
                                      const void* v_pool, const void* q, void* out,
                                      pa_dtype out_dtype, const int32_t* q_start,
                                      const int32_t* block_tables, int32_t max_blocks_per_seq,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_q_heads, float scale, int32_t max_chunk_len,
                                      int32_t max_context_len, void* stream);

/* Directions of pa_swap_blocks. */
enum { PA_SWAP_OUT = 0, PA_SWAP_IN = 1 };

/*
 * pa_swap_blocks -- preemption by swapping: copy whole blocks (every slot,
 * both pools, all KV heads) between the device pools and host pools of the
 * same layout.  When the pool is exhausted a whole sequence is evicted and
 * its K/V moved to CPU memory, to be restored later (transcript, paragraph
 * 5); the cost is the cache bytes in each direction ("Inside vLLM and TGI",
 * section "Read the vLLM0.11.0 scheduler").
 *   host_k, host_v    HOST, page-locked (hipHostMalloc or an equivalent pinned
 *                     allocation) and mapped for the current device: host
 *                     block hb starts at byte hb * Hkv * b * head_dim * s; the
 *                     GPU reads or writes them directly (no staging copy)
 *   host_num_blocks   blocks in each host pool
 *   block_pairs       device int32 [n_pairs][2] (src, dst): for PA_SWAP_OUT
 *                     (device block, host block), for PA_SWAP_IN (host block,
 *                     device block); a pair with an id out of range is skipped;
 *                     no block may be the destination of two pairs
 *   direction         PA_SWAP_OUT or PA_SWAP_IN
 * Host pools that are not pinned host memory are rejected (PA_ERR_INVALID_ARG)
 * before anything is enqueued.  The host data is complete once the stream has
 * passed the call.
 */
PA_API pa_status pa_swap_blocks(const pa_pool_desc* pool, void* k_pool, void* v_pool,
                                void* host_k, void* host_v, int32_t host_num_blocks,
                                const int32_t* block_pairs, int32_t n_pairs, int32_t direction,
                                void* stream);

/*
 * pa_validate_tables -- debug check of device-resident tables before a
 * kernel consumes them ("Inside vLLM and TGI", section "Exact CPU block
 * manager and copy-on-write", validation paragraph).  Counts violations:
 * a length outside [1, min(max_context_len, max_blocks_per_seq * b)], or a
 * table entry j < ceil(L_i / b) outside [0, num_blocks).
 *   bad_count   device int32 [1] (output): number of violations
 * Asynchronous like every other call; read bad_count after the stream passes.
 */
PA_API pa_status pa_validate_tables(const pa_pool_desc* pool, const int32_t* block_tables,
                             int32_t max_blocks_per_seq, const int32_t* context_lens,
                             int32_t num_seqs, int32_t max_context_len, int32_t* bad_count,
                             void* stream);

/*
 * pa_validate_copy_pairs -- debug check of one pa_copy_blocks batch against
 * its contract.  A copy-on-write fills a block just taken from the free list
 * with the old block's contents ("Inside vLLM and TGI", section "Exact CPU
 * block manager and copy-on-write"; transcript paragraph 4), so a batch of
 * copies issued at once means the same as the copies one after another only
 * when every destination is distinct and none is also a source.  Counts the
 * pairs that break this: pair i counts once when its destination is the
 * destination of another pair or the source of any pair (its own included).
 * Pairs with an id outside [0, num_blocks) are skipped by pa_copy_blocks and
 * take no part.
 *   block_pairs  device int32 [n_pairs][2] = {src, dst}
 *   bad_count    device int32 [1] (output): number of offending pairs
 * n_pairs^2 comparisons on the device (meant for debug batches).
 * Asynchronous like every other call; read bad_count after the stream passes.
 */
PA_API pa_status pa_validate_copy_pairs(const pa_pool_desc* pool, const int32_t* block_pairs,
                                        int32_t n_pairs, int32_t* bad_count, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_H */
