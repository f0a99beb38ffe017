/*
 * pkv.h -- C ABI of libpkv.so: paged KV-cache decode attention on AMD
 * Instinct MI355X (gfx950).
 *
 * What is computed comes from three web pages on paged KV caches:
 *  [ttlab]  "Basics of LLM Inference and vLLM Internals: KV Cache,
 *           PagedAttention, and Scheduler" -- section 2 (sizing formula,
 *           MQA/GQA, fp8 KV) and section 4 (16-token blocks, per-request
 *           block table, physical block pool, shared prefix blocks,
 *           reserved null block 0).
 *  [redhat] drpranayjha, "How PagedAttention pages the KV cache" (fixed
 *           16-token blocks, block table to non-adjacent physical blocks,
 *           waste only in the last block, shared prefixes).
 *  [tarun]  tarundecipher, "The Memory Trick Behind Fast LLM Serving" --
 *           "PagedAttention changes the shape of the problem" and "Batching
 *           does not merge the conversations" (a flattened batch whose
 *           metadata keeps each sequence's context private).
 *
 * Conventions (all entry points)
 *  - Every function returns an int status: PKV_OK or a negative PKV_ERR_*.
 *    pkv_status_string() names it.
 *  - All buffers are caller-owned, contiguous, row-major device memory
 *    unless a parameter says "host". The library allocates no memory and
 *    keeps no state between calls beyond what it sets up once per device
 *    (the compute-unit count and each decode kernel's occupancy), and is
 *    safe to call from several host threads.
 *  - Work is enqueued on the given HIP stream (NULL = the null stream) and
 *    never synchronised: results are visible after the stream reaches the
 *    point of the call. No call issues a memset, a copy or a host
 *    synchronisation, and workspaces keep their counters at zero from call
 *    to call, so a sequence of calls may be captured in a HIP graph and
 *    replayed (with the same buffers, which replays reuse).
 *  - Argument errors that the host can see (null pointers, sizes, dtypes)
 *    return before any HIP call; launch failures return PKV_ERR_HIP.
 *  - Values in device memory (block ids, slots, lengths) are not read by the
 *    host. Out-of-range ones never cause an out-of-bounds access: the
 *    kernels skip such slots and turn such sequences into NaN rows, as
 *    documented per call.
 *
 * KV cache layout (one tensor each for K and V, same size):
 *     num_blocks * num_kv_heads * 16 * head_dim elements.
 * One (block, KV head) tile -- the 16 token rows of that block for that KV
 * head, 16 * head_dim elements -- is contiguous, tile (blk, g) first element
 * at (blk * num_kv_heads + g) * 16 * head_dim. Inside a tile, row `off`
 * (0..15), element j (0..head_dim-1) is at
 *     K: ((j / 8) * 16 + off) * 8 + j % 8    (8-element slabs, token-minor)
 *     V: (((j / 32) * 16 + j % 16) * 4 + off / 4) * 8 + ((j / 16) % 2) * 4 + off % 4
 *        (runs of 4 consecutive rows of one element, two element blocks of
 *        16 interleaved)
 * an order chosen so that the decode kernel's matrix-core operands load as
 * contiguous runs. Only the library writes this order (pkv_kv_append) and
 * reads it (decode, pkv_debug_gather): callers pass whole rows in and get
 * whole rows out, and need the layout only to size the tensors.
 * Token position t of a sequence lives in physical block
 * block_tables[s][t / 16], row t % 16 ([ttlab] section 4: logical block ->
 * physical block through the request's block table). A slot is the flat row
 * index phys_block * 16 + row.
 */
#ifndef PKV_H
#define PKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Same definition as HIP's own, so the header needs no HIP include. */
typedef struct ihipStream_t *hipStream_t;

/* Status codes. */
#define PKV_OK 0
#define PKV_ERR_INVALID_ARG (-1) /* null pointer, non-positive size, bad ratio */
#define PKV_ERR_UNSUPPORTED (-2) /* valid but not built: dtype pair, head_dim, group */
#define PKV_ERR_WORKSPACE (-3)   /* workspace missing or smaller than required */
#define PKV_ERR_HIP (-4)         /* a HIP launch reported an error */
#define PKV_ERR_TOO_LARGE (-5)   /* beyond the allocation-free entry point's static scratch */

/* Element types. PKV_FP8_E4M3 is OCP E4M3FN: 1 sign, 4 exponent bits
 * (bias 7), 3 mantissa bits, no infinities, NaN = 0x7F / 0xFF, largest
 * finite 448 ([ttlab] sections 2 and 7: an fp8 KV cache, b = 1). An fp8
 * element's value is code * scale with one float scale per tensor. */
typedef enum {
    PKV_F32 = 0,
    PKV_F16 = 1,
    PKV_BF16 = 2,
    PKV_FP8_E4M3 = 3
} pkv_dtype;

/* The tokens of one physical block ([ttlab] section 4, [redhat]). The only
 * block size this library accepts. */
#define PKV_BLOCK_SIZE 16

/* Describes both k_cache and v_cache (see the layout above).
 *  num_blocks    physical blocks in the pool (> 0)
 *  block_size    must be PKV_BLOCK_SIZE
 *  num_kv_heads  H_kv (> 0)
 *  head_dim      d: 64 or 128
 *  dtype         element type of both caches
 *  k_scale, v_scale  per-tensor scales for PKV_FP8_E4M3 (ignored otherwise) */
typedef struct {
    int32_t num_blocks;
    int32_t block_size;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t dtype; /* a pkv_dtype */
    float k_scale;
    float v_scale;
} pkv_cache_desc;

/* Text for a status code (static storage, never NULL). */
const char *pkv_status_string(int status);

/* KV bytes per token over the whole model: 2 (K and V) * num_layers *
 * num_kv_heads * head_dim * element bytes ([ttlab] section 2, the sizing
 * formula; [redhat] "How PagedAttention pages the KV cache", the 40-layer
 * example). Returns 0 for a non-positive size or an unknown dtype. */
size_t pkv_kv_bytes_per_token(int32_t num_layers, int32_t num_kv_heads, int32_t head_dim,
                              int32_t dtype);

/* Bytes of ONE cache tensor (K or V) described by *cache:
 * num_blocks * num_kv_heads * 16 * head_dim * element bytes. 0 if invalid. */
size_t pkv_cache_tensor_bytes(const pkv_cache_desc *cache);

/* Slot-mapped append: write each new token's K and V rows into its block.
 * ([ttlab] section 4: physical blocks are filled one token row at a time as
 * a request grows; the block-table figure shows a last block 6/16 full.)
 *
 *  k, v          [num_tokens][num_kv_heads][head_dim] in kv_dtype (device)
 *  kv_dtype      equal to cache->dtype: the rows are copied byte for byte.
 *                Or PKV_F32 / PKV_F16 / PKV_BF16 into a PKV_FP8_E4M3 cache
 *                ([ttlab] section 2: fp8 storage, one byte per element):
 *                element x of K is stored as the E4M3FN code of the float32
 *                quotient x / cache->k_scale (one IEEE single-precision
 *                division, round to nearest even), V likewise with v_scale;
 *                the code is the nearest one, ties to an even mantissa,
 *                quotients beyond +-448 (and infinities) saturate to +-448,
 *                NaN becomes 0x7F.
 *  slot_mapping  int64 [num_tokens] (device). Token i goes to block
 *                slot / 16, row slot % 16, for every KV head (stored in the
 *                in-tile order above; filling every slot of a pool from
 *                row-order data is how a caller builds a cache). A negative
 *                slot skips the token; a slot >= num_blocks * 16 is also
 *                skipped (precondition violation, never written).
 *  num_tokens    >= 0 (0 is a no-op that still validates)
 *  k_cache, v_cache  the pool tensors (device), updated in place
 * Two tokens with the same slot in one call race (precondition: distinct).
 * Errors: INVALID_ARG (null pointer with num_tokens > 0, bad desc),
 * UNSUPPORTED (block size, head_dim, dtype, a kv_dtype / cache dtype pair
 * other than the above), HIP. */
int pkv_kv_append(const void *k, const void *v, int32_t kv_dtype, const int64_t *slot_mapping,
                  int32_t num_tokens, void *k_cache, void *v_cache, const pkv_cache_desc *cache,
                  hipStream_t stream);

/* Largest number of worker waves one decode launch uses. */
#define PKV_MAX_WORKERS 4096

/* Workspace bytes pkv_paged_attention_decode needs for this batch shape,
 * partition size and worker count. Gp is G = num_q_heads / num_kv_heads
 * rounded up to 1, 2, 4, 6 or 8, and one partial slot holds Gp * head_dim +
 * pad(2 * Gp) floats (an accumulator row, a maximum and a sum per head;
 * pad() rounds up to a multiple of 4). Front, float partial slots:
 *   partition_size == 0 (balanced split): 2 * workers slots, workers =
 *     num_workers or PKV_MAX_WORKERS for num_workers 0;
 *   partition_size  > 0 (fixed partitions): one slot per (sequence, KV head,
 *     partition), num_seqs * num_kv_heads * Pn slots with
 *     Pn = ceil(max_blocks_per_seq * 16 / partition_size); for G = 2, 4, 6
 *     or 8 that is num_seqs * num_q_heads * Pn * (head_dim + 2) floats.
 * End: int32 counters [num_seqs][num_kv_heads]. Each part is rounded up to
 * 256 bytes. Returns 0 for invalid arguments (non-positive sizes, G not a
 * whole number or above 8, a partition size that is negative or not a
 * multiple of 16, num_workers < 0 or > PKV_MAX_WORKERS).
 *
 * Workspace rule (both decode entry points): the counters sit in the last
 * bytes of the workspace as passed (workspace_bytes rounded down to 256) and
 * must be zero when a call starts; every call leaves them zero. Float
 * scratch sits at the front. So a workspace sized for the largest shape a
 * caller runs (num_seqs, max_blocks_per_seq, num_groups, num_workers; same
 * heads, head_dim and partition size) and zeroed once serves any call of
 * that shape or smaller, passed with the same workspace_bytes, without being
 * cleared again. */
size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t max_blocks_per_seq,
                                  int32_t partition_size, int32_t num_workers);

/* Paged decode attention: one new query token per sequence attends over its
 * own cached tokens, read through its block table.
 * ([ttlab] section 4 and [redhat]: block table lookup into a shared pool;
 *  [ttlab] section 2: query head h of H_q shares KV head h / (H_q / H_kv)
 *  (GQA, MQA when H_kv = 1); [tarun] "Batching does not merge the
 *  conversations": sequences in one batch never see each other's blocks.)
 *
 * For sequence s with n = context_lens[s] and query head h, g = h / G:
 *     x_t = scale * (q[s][h] . K_t),  t in [0, n),  K_t = k_cache row of t
 *     out[s][h] = sum_t exp(x_t - max_u x_u) * V_t / sum_t exp(x_t - max_u x_u)
 * with fp8 elements read as code * k_scale / code * v_scale. n counts the
 * query's own token, whose K/V must already be appended. n <= 0 gives a zero
 * row. Arithmetic is float32; the result is rounded to nearest-even into
 * q_dtype.
 *
 * Split-KV, two ways (results depend on the split only through float32
 * rounding, and are bit-for-bit repeatable for a fixed split and device):
 *  - partition_size == 0, the balanced split: the (sequence, KV head,
 *    16-token block) tiles of the whole batch are split evenly over
 *    num_workers waves, so a long (sequence, KV head) may be shared by
 *    several waves; each leaves a partial (max, sum, accumulator) and the
 *    last one to finish merges them by the log-sum-exp rule.
 *  - partition_size = P > 0, fixed partitions: the tokens of each (sequence,
 *    KV head) are cut into partitions [j * P, min((j + 1) * P, n)); the
 *    partitions of the batch are split evenly over num_workers waves (whole
 *    partitions each); every partition of a sequence with more than one
 *    leaves its partial (max, sum, accumulator) in its own workspace slot,
 *    and a second launch on the stream reduces them by the log-sum-exp rule
 *    (one wave per sequence and query head).
 *
 *  q             [num_seqs][num_q_heads][head_dim] in q_dtype (device)
 *  q_dtype       (q, cache) pairs: (F32, F32), (F16, F16), (BF16, BF16),
 *                (F16 or BF16, FP8_E4M3)
 *  num_q_heads   H_q, a multiple of cache->num_kv_heads with G = H_q / H_kv
 *                at most 8
 *  block_tables  int32 [num_seqs][max_blocks_per_seq] (device); only the
 *                first ceil(n / 16) entries of a row are read
 *  context_lens  int32 [num_seqs] (device)
 *  scale         softmax scale applied to q . k (typically 1/sqrt(head_dim))
 *  partition_size  0 (balanced split) or tokens per fixed partition, a
 *                positive multiple of 16
 *  num_workers   waves sharing the work: 0 = enough to fill the device (with
 *                fixed partitions: the waves that give every wave about the
 *                same whole number of partitions of a batch of full-length
 *                sequences), otherwise 1..PKV_MAX_WORKERS
 *  workspace, workspace_bytes  at least pkv_decode_workspace_bytes(...) of
 *                device memory, 256-byte aligned, zeroed before its first
 *                use (see the workspace rule above). Two calls must not use
 *                one workspace at the same time.
 *  out           [num_seqs][num_q_heads][head_dim] in q_dtype (device); must
 *                not alias any input or the workspace
 * A sequence whose length exceeds max_blocks_per_seq * 16, or whose needed
 * block ids fall outside [0, num_blocks), gets a NaN row (no out-of-range
 * read happens). Errors: INVALID_ARG (also a partition size that is negative
 * or not a multiple of 16), UNSUPPORTED, WORKSPACE, HIP. */
int pkv_paged_attention_decode(const void *q, int32_t q_dtype, int32_t num_seqs,
                               int32_t num_q_heads, const void *k_cache, const void *v_cache,
                               const pkv_cache_desc *cache, const int32_t *block_tables,
                               int32_t max_blocks_per_seq, const int32_t *context_lens,
                               float scale, int32_t partition_size, int32_t num_workers,
                               void *workspace, size_t workspace_bytes, void *out,
                               hipStream_t stream);

/* Bytes of the static device scratch array behind
 * pkv_paged_attention_decode_noalloc (one per GPU the library runs on, held
 * until the process ends). */
#define PKV_NOALLOC_SCRATCH_BYTES (48u << 20)

/* pkv_paged_attention_decode without a workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc. The call allocates nothing (no
 * hipMalloc, hipFree or allocating library routine): its workspace is a
 * static device array of PKV_NOALLOC_SCRATCH_BYTES, one per GPU, whose
 * device address is taken on the first call on that GPU (make that first
 * call outside a graph capture). Each call first zeroes the counters it uses
 * (a small kernel on the stream, no memset), then runs the same decode
 * kernel as pkv_paged_attention_decode, so for the same arguments the output
 * is bit-for-bit the same.
 * All arguments, results and errors as for pkv_paged_attention_decode, plus
 * PKV_ERR_TOO_LARGE (before any HIP call) when
 * pkv_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
 * max_blocks_per_seq, partition_size, num_workers) exceeds
 * PKV_NOALLOC_SCRATCH_BYTES. Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (other streams, other host threads) race and
 * must be serialised by the caller. */
int pkv_paged_attention_decode_noalloc(const void *q, int32_t q_dtype, int32_t num_seqs,
                                       int32_t num_q_heads, const void *k_cache,
                                       const void *v_cache, const pkv_cache_desc *cache,
                                       const int32_t *block_tables, int32_t max_blocks_per_seq,
                                       const int32_t *context_lens, float scale,
                                       int32_t partition_size, int32_t num_workers, void *out,
                                       hipStream_t stream);

/* Workspace bytes pkv_paged_attention_decode_shared_prefix needs. Front:
 * the decode slots for the worker count, float32 suffix results
 * (num_seqs * num_q_heads * head_dim, then num_seqs * num_q_heads floats) and
 * 4096 prefix partial slots of 16 * head_dim + 32 floats. End: the decode
 * counters [num_seqs][num_kv_heads]. Each part is rounded up to 256
 * bytes. Returns 0 where pkv_decode_workspace_bytes does, or for
 * num_groups < 0 or > num_seqs. */
size_t pkv_shared_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t num_groups, int32_t num_workers);

/* Paged decode for a batch whose sequences share prefixes: the same result
 * as pkv_paged_attention_decode with the same arguments (up to float32
 * rounding order), reading each shared block once per KV head for all the
 * sequences that reference it instead of once per sequence.
 * ([ttlab] section 4 and [redhat]: sequences with a common prefix map its
 *  logical blocks to one physical copy, listed in each of their block
 *  tables.)
 *
 * Prefix groups (device arrays, read by the kernels only):
 *  group_starts         int32 [num_groups + 1]: group j is the run of
 *                       sequences [group_starts[j], group_starts[j + 1])
 *  group_prefix_blocks  int32 [num_groups]: P_j, the number of leading
 *                       logical blocks that every member of group j maps to
 *                       the same physical blocks (full blocks: 16 * P_j
 *                       tokens)
 * Preconditions: every member's first P_j block-table entries equal those of
 * the group's first sequence (the library reads the group's blocks from that
 * row), and every member's context_lens holds them (n >= 16 * P_j). A member
 * with n < 16 * P_j, or longer than max_blocks_per_seq * 16, gets a NaN row.
 * Sequences outside every group, and groups with P_j = 0, are decoded as by
 * pkv_paged_attention_decode. The description is used only as a whole: if
 * group_starts is not non-decreasing inside [0, num_seqs] or some P_j lies
 * outside [0, max_blocks_per_seq], it is ignored and every sequence is
 * decoded plainly (still the same result).
 *
 * How: three launches. The suffix pass is the decode kernel over each
 * member's blocks after its group's prefix; it leaves the members' rows as
 * float32 (normalised output, log2-sum-exp) in the workspace. The prefix
 * pass stacks the (member, query head) rows of a group 128 to a workgroup
 * against the shared tiles, read once per workgroup through LDS, and splits
 * the prefix into chunks when there are few rows. When every 16-row block of
 * the batch can hold a partial slot (num_kv_heads * (ceil(num_seqs * G / 16)
 * + num_groups) <= 4096), the prefix pass leaves all its partials in the
 * workspace and runs beside the suffix pass: one launch on `stream` whose
 * workgroups take either pass. Otherwise it runs after the suffix pass on
 * `stream`, merging one-chunk groups with their suffix results itself. The
 * merge launch on `stream` then combines the chunk partials with the suffix
 * results by the log-sum-exp rule into out.
 *
 *  num_groups   0..num_seqs (0: plain decode; the arrays may then be NULL)
 *  workspace    at least pkv_shared_prefix_workspace_bytes(...) bytes,
 *               256-byte aligned, zeroed before its first use (the
 *               workspace rule above). One call at a time.
 * All other arguments as for pkv_paged_attention_decode. Errors: as for
 * pkv_paged_attention_decode, plus INVALID_ARG for num_groups outside
 * [0, num_seqs] or a NULL group array with num_groups > 0. */
int pkv_paged_attention_decode_shared_prefix(
    const void *q, int32_t q_dtype, int32_t num_seqs, int32_t num_q_heads, const void *k_cache,
    const void *v_cache, const pkv_cache_desc *cache, const int32_t *block_tables,
    int32_t max_blocks_per_seq, const int32_t *context_lens, int32_t num_groups,
    const int32_t *group_starts, const int32_t *group_prefix_blocks, float scale,
    int32_t num_workers, void *workspace, size_t workspace_bytes, void *out, hipStream_t stream);

/* Paged chunked-prefill attention: each sequence brings a chunk of new query
 * tokens that attend causally to its cached tokens, read through its block
 * table ([ttlab] section 6: a prompt longer than the per-step token budget is
 * processed in chunks; section 4: the paged cache).
 *
 * Sequence s owns query rows [query_start[s], query_start[s + 1]) of q: its
 * q_len newest tokens, whose K/V are already appended, so that with
 * n = context_lens[s] token i of the chunk sits at position p = n - q_len + i.
 * For query head h (KV head g = h / G):
 *     out[query_start[s] + i][h] = sum_{t <= p} exp(x_t - max) V_t / sum_{t <= p} exp(x_t - max),
 *     x_t = scale * (q[query_start[s] + i][h] . K_t)
 * (fp8 elements read as code * k_scale / code * v_scale). One query token per
 * sequence is decode. Arithmetic is float32 on the matrix cores; the result
 * is rounded to nearest-even into q_dtype.
 *
 *  q, out        [num_tokens][num_q_heads][head_dim] in q_dtype (device)
 *  query_start   int32 [num_seqs + 1] (device), non-decreasing from 0 to
 *                num_tokens
 *  block_tables, context_lens, scale, q_dtype / cache pairs: as for decode
 * A sequence whose chunk is not inside [0, num_tokens], is longer than its
 * context, or whose context exceeds max_blocks_per_seq * 16 is skipped (its
 * rows are not written); one whose needed block ids fall outside the pool gets
 * NaN rows.
 *
 *  workspace, workspace_bytes  NULL (each 128-row tile of a sequence is one
 *                workgroup over all its keys), or at least
 *                pkv_prefill_workspace_bytes(head_dim) bytes of device memory,
 *                256-byte aligned (no zeroing needed). With a workspace, a
 *                batch with few rows (short chunks over long contexts) splits
 *                each row tile's keys into chunks computed by separate
 *                workgroups, and a second launch merges the chunk partials
 *                (float32 m, l and accumulators) by the log-sum-exp rule. One
 *                call at a time per workspace.
 * Errors: INVALID_ARG, UNSUPPORTED (as decode, or a batch too large for one
 * launch), WORKSPACE (misaligned or too small), HIP. */
int pkv_paged_attention_prefill(const void *q, int32_t q_dtype, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_q_heads,
                                const int32_t *query_start, const void *k_cache,
                                const void *v_cache, const pkv_cache_desc *cache,
                                const int32_t *block_tables, int32_t max_blocks_per_seq,
                                const int32_t *context_lens, float scale, void *workspace,
                                size_t workspace_bytes, void *out, hipStream_t stream);

/* Workspace bytes for pkv_paged_attention_prefill's key split: 4096 partial
 * slots of 16 rows (16 * head_dim + 32 floats each), rounded up to 256. 0 for
 * a head_dim other than 64 or 128. */
size_t pkv_prefill_workspace_bytes(int32_t head_dim);

/* Copy whole physical blocks, every KV head of K and V:
 *     block pairs[i][1] <- block pairs[i][0],   i < num_pairs.
 * The copy-on-write step ([ttlab] section 4): before a request appends into a
 * block it shares with others, the block is copied and the request's table
 * points at the copy. The block manager (pkv_blocks.h) emits the pairs.
 *  pairs  int32 [num_pairs][2] (device); a pair with an id outside
 *         [0, num_blocks) is skipped. A destination that is also a source, or
 *         two pairs with one destination, in one call race.
 * Errors: INVALID_ARG (null pointer with num_pairs > 0, negative count,
 * misaligned cache, bad desc), UNSUPPORTED, HIP. */
int pkv_copy_blocks(void *k_cache, void *v_cache, const pkv_cache_desc *cache,
                    const int32_t *pairs, int32_t num_pairs, hipStream_t stream);

/* Gather through the block tables (the same device addressing code as the
 * decode kernel), for checking indexing byte for byte:
 *     k_out[s][g][t][:] = K row of position t of sequence s, KV head g
 * for t < min(context_lens[s], max_ctx); other rows of k_out/v_out are left
 * untouched. k_out, v_out: [num_seqs][num_kv_heads][max_ctx][head_dim] in
 * the cache dtype (device). Sequences with invalid lengths or block ids are
 * skipped entirely. Errors: INVALID_ARG, UNSUPPORTED, HIP. */
int pkv_debug_gather(const void *k_cache, const void *v_cache, const pkv_cache_desc *cache,
                     const int32_t *block_tables, int32_t max_blocks_per_seq,
                     const int32_t *context_lens, int32_t num_seqs, int32_t max_ctx, void *k_out,
                     void *v_out, hipStream_t stream);

/* Measurement helper, not part of the attention path: read `bytes` of
 * device memory at `src` once as a plain stream of 16-byte nontemporal
 * loads (the decode kernel's load width and cache policy), spread over
 * num_workgroups workgroups of 256 threads (0 = one per compute unit), and XOR
 * every 32-bit word into *sink (device; one atomic per workgroup) so that no read
 * can be dropped. Timed by the caller, it gives the read bandwidth this
 * device delivers to a streaming kernel: the yardstick beside the published
 * HBM peak ([ttlab] section 1 judges decode by the fraction of the rated
 * bandwidth it reaches).
 *  src   device, 16-byte aligned; bytes a multiple of 16 (0: nothing to do)
 *  sink  device uint32, 4-byte aligned; XORed into, never cleared
 * Errors: INVALID_ARG (null pointer, misalignment, negative count), HIP. */
int pkv_stream_read(const void *src, size_t bytes, uint32_t *sink, int32_t num_workgroups,
                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PKV_H */
