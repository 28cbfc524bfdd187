/*
 * pagedattn.h -- C ABI of the MI355X (gfx950) paged KV-cache attention library.
 *
 * The method: the KV cache is cut into fixed-size blocks that sit anywhere in
 * one shared pool; each sequence finds its blocks through a block table that
 * maps logical positions to physical blocks, and the attention kernel reads
 * the scattered blocks directly, with no contiguous copy ("Ultimate Guide to
 * PagedAttention", newline: KV blocks, block table, non-contiguous storage;
 * Kwon et al., "Efficient Memory Management for Large Language Model Serving
 * with PagedAttention", abstract; Joshi et al., "Paged Attention Meets
 * FlexAttention", abstract: a fused kernel that gathers the scattered KV
 * data).  The result is exact softmax attention (Dao et al., "FlashAttention",
 * abstract), optionally with FlexAttention-style mask/score modification.
 *
 * ---------------------------------------------------------------------------
 * Storage (device memory, owned by the caller)
 *
 *   element type   PA_F32 (float) or PA_BF16 (bfloat16 bits); q, the pools,
 *                  new tokens and outputs of one call share it.  Arithmetic
 *                  accumulates in fp32.
 *   k_cache        [num_blocks, num_kv_heads, block_size, head_dim]
 *                  (token-major rows inside each (block, kv-head) slab)
 *   v_cache        [num_blocks, num_kv_heads, block_size / 16, head_dim, 16]
 *                  (dimension-major sub-slabs of 16 tokens: token o of a
 *                  block is column o % 16 of sub-slab o / 16, so any 16-token
 *                  chunk's values are one contiguous run for every page size)
 *   block_tables   int32 [num_seqs, block_table_stride]; entry [b, j] is the
 *                  physical block of logical tokens [j*bs, (j+1)*bs) of
 *                  sequence b.  Only entries j < ceil(context_lens[b]/bs) are
 *                  read.
 *   context_lens   int32 [num_seqs]: keys of sequence b (including tokens
 *                  appended for this step).  Key j sits at logical position j.
 *   query row i of a sequence with n keys and L query rows sits at logical
 *   position n - L + i (decode: L = 1, position n - 1).  Query head h reads
 *   kv-head h / (num_heads / num_kv_heads).
 *
 * Tensor pointers (q, out, the pools, new tokens, workspaces) must be 16-byte
 * aligned: the kernels move 16-byte pieces.  All calls are asynchronous on
 * `stream` (a hipStream_t; NULL = the null stream).  No call allocates device
 * or host memory.  None keeps state between calls, except the per-device
 * scratch of paged_attn_decode_noalloc, and calls are thread-safe, except
 * paged_attn_decode_noalloc calls that overlap on one device.
 *
 * Status: 0 = success.  A negative value is an invalid argument found on the
 * host before anything is enqueued (no buffer is touched).  A positive value
 * is the hipError_t of a failed launch.  paged_attn_status_string() names
 * every code.
 *
 * Device contents are not validated (that would need a device->host sync):
 * block ids must lie in [0, num_blocks), context_lens[b] must not exceed
 * block_table_stride * block_size, a prefill sequence must have
 * q_len <= context_len, and the slots of one kv_append must be distinct.
 * Breaking these is undefined behaviour in the release library; the same
 * library built with PA_DEBUG_CHECKS (libpagedattn_debug.so) checks block
 * ids and lengths on the device and traps instead.
 * ---------------------------------------------------------------------------
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

enum {
  PA_OK = 0,
  PA_ERR_NULL = -1,          /* a required pointer is NULL                      */
  PA_ERR_SIZE = -2,          /* a count is negative or exceeds the index range   */
  PA_ERR_HEADS = -3,         /* heads <= 0, or num_heads % num_kv_heads != 0     */
  PA_ERR_HEAD_DIM = -4,      /* head_dim not 64 or 128                          */
  PA_ERR_BLOCK_SIZE = -5,    /* block_size not a power of two in [16, 256]      */
  PA_ERR_SPLIT = -6,         /* split_tokens not 0, -1, -2 or a power of two >= 16;
                                key_split not 0, -1 or a multiple of 64 */
  PA_ERR_WORKSPACE = -7,     /* workspace NULL or smaller than required         */
  PA_ERR_DTYPE = -8,         /* dtype not PA_F32 / PA_BF16                      */
  PA_ERR_FLAG = -9,          /* causal not 0 or 1                               */
  PA_ERR_MODS = -10,         /* window < 0, softcap < 0 or not finite, or a bad
                                block mask                                      */
  PA_ERR_TABLE_STRIDE = -11, /* block_table_stride < 1                          */
  PA_ERR_NO_BLOCKS = -12,    /* block manager: the pool is exhausted            */
  PA_ERR_SEQ = -13,          /* block manager: unknown or freed sequence id     */
  PA_ERR_ALIGN = -14,        /* a tensor pointer is not 16-byte aligned         */
  PA_ERR_SCRATCH = -15       /* paged_attn_decode_noalloc: needs more than
                                PA_DECODE_SCRATCH_BYTES of workspace            */
};

/*
 * FlexAttention-style modifications on logical positions (Joshi et al.,
 * "Paged Attention Meets FlexAttention", abstract: the paged kernel keeps
 * FlexAttention's programmable masks and score mods).  With s = scale * q.k:
 *   softcap > 0   : s = softcap * tanh(s / softcap)
 *   alibi_slopes  : s = s + alibi_slopes[h] * (key_pos - query_pos)
 *                   (device pointer to num_heads floats; NULL = none)
 *   window > 0    : keys with query_pos - key_pos >= window are masked out
 *   prefix_lens   : prefix-LM; with causal masking, keys at positions below
 *                   prefix_lens[b] are seen by every row of sequence b
 *                   (device pointer to num_seqs int32; NULL = none)
 *   doc_starts    : document masking of packed sequences; keys before
 *                   doc_starts[row] are masked out for that query row
 *                   (device pointer, one int32 per query row -- num_seqs for
 *                   decode, total_q for prefill; NULL = none)
 *   block_mask    : FlexAttention-style block sparsity (pa_block_mask below):
 *                   which key blocks each query block sees at all; the other
 *                   masks still apply inside the blocks it admits (NULL =
 *                   none)
 * Masks only shrink a row's key range, so fully masked key tiles are never
 * read.  Passing NULL for the struct means none of them.  The structs
 * themselves are read on the host during the call and may be freed on
 * return.
 */
/*
 * A block mask: for sequence b and a query at logical position p, bitmap row
 * b * rows_per_seq + p / q_block of `bits` (device uint32 [num_seqs *
 * rows_per_seq, words_per_row]) admits key j only if bit (j / kv_block) % 32
 * (bit 0 = least significant) of word (j / kv_block) / 32 is set.  q_block is
 * a power of two >= 1, kv_block a power of two in [64, 2^24] (whole 64-key
 * tiles of the prefill kernel), rows_per_seq and words_per_row >= 1
 * (PA_ERR_MODS otherwise).  Caller contract (not checked on the device): every
 * row and word that a query's position and a sequence's keys address exist.
 * Key blocks no row of a work-group admits are never read; a decode row skips
 * the 16-token chunks of blocks it does not admit.  Reading of "Paged
 * Attention Meets FlexAttention" (abstract): the paged kernel keeps
 * FlexAttention's programmable masks, of which the block mask is the one that
 * saves work.
 */
typedef struct {
  const uint32_t* bits;
  int32_t q_block;
  int32_t kv_block;
  int32_t rows_per_seq;
  int32_t words_per_row;
} pa_block_mask;

typedef struct {
  int32_t window;
  float softcap;
  const float* alibi_slopes;
  const int32_t* prefix_lens;
  const int32_t* doc_starts;
  const pa_block_mask* block_mask;
} pa_score_mods;

/*
 * kv_append -- store the key/value vectors of new tokens in the paged cache.
 *
 * New tokens' vectors are written into the blocks a growing sequence owns;
 * existing data never moves ("Ultimate Guide to PagedAttention": KV cache,
 * dynamic growth).  For every t < num_tokens with s = slot_mapping[t] >= 0:
 *   k_cache[s / bs][h][s % bs][:] = k_new[t][h][:]
 *   v_cache[s / bs][h][(s % bs) / 16][:][s % 16] = v_new[t][h][:]
 * for every kv-head h.
 * Tokens with a negative slot are skipped.  The copy is bit-exact (no
 * conversion).  k_new / v_new: [num_tokens, num_kv_heads, head_dim].
 * num_tokens == 0 is a no-op.
 */
int kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
              const int32_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
              int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t dtype,
              void* stream);

/*
 * kv_copy_blocks -- copy whole physical blocks (copy-on-write, fork).
 *
 * For every i < num_pairs and every kv-head, the K slab and the V slab of
 * block src_blocks[i] are copied bit for bit onto block dst_blocks[i]
 * ("Ultimate Guide to PagedAttention": copy-on-write when a shared block is
 * written).  src_blocks / dst_blocks: device int32 [num_pairs].  Caller
 * contract (not checked on the device): ids in [0, num_blocks), no
 * destination listed twice and no destination that is also a source.
 * num_pairs == 0 is a no-op.
 */
int kv_copy_blocks(void* k_cache, void* v_cache, const int32_t* src_blocks, const int32_t* dst_blocks,
                   int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                   int64_t num_blocks, int32_t dtype, void* stream);

/*
 * Bytes of workspace paged_attn_decode needs for these sizes.  Split-KV --
 * cutting a row's context into pieces whose partial softmax states (output,
 * running max, running sum) are merged afterwards -- is this library's
 * reading of how to spread long decode rows over many compute units; the
 * pages only motivate long contexts.  split_tokens:
 *    0  the library's choice, from the sizes alone:
 *       - max_context_len <= 256: no row is split (no merge launch);
 *       - else, while num_seqs * num_kv_heads * ceil(max_context_len / 512)
 *         is at most 16 per compute unit: fixed pieces of 512 keys,
 *         longer (powers of two) when a row would hold more than 32 of them
 *         (a small batch finishes sooner on these than on the balanced
 *         split);
 *       - else the balanced split (-2);
 *   -2  balanced split: 8 wavefronts per compute unit of the current device
 *       (256 units if none is visible) each take an equal share of the
 *       batch's 16-token chunks, at least 8, so the pieces follow the work,
 *       not a fixed length (batches of more than 4096 sequences take fixed
 *       pieces instead);
 *   -1  never split;
 *  > 0  fixed pieces of split_tokens keys (a power of two >= 16).
 * Fixed pieces of at least 64 keys run as 4-wavefront work-groups when the
 * whole grid fits on the device at once (two per compute unit).
 * Returns 0 for invalid arguments.
 */
size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t max_context_len, int32_t split_tokens);

/* The split paged_attn_decode will use: 0 for the balanced split, -1 for
 * none, else the fixed piece length (0 also for invalid arguments). */
int32_t paged_attn_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                       int32_t max_context_len, int32_t split_tokens);

/*
 * paged_attn_decode -- one query row per sequence over its paged context.
 *
 * The decode step of serving: each sequence's newest token attends to every
 * key its blocks hold, read where the blocks lie through the block table
 * ("Ultimate Guide to PagedAttention": block table, non-contiguous storage;
 * Kwon et al., abstract: attention over non-contiguous KV blocks).  The
 * pages note that this step is bound by loading the KV cache (the vAttention
 * page's decode snippet), so the kernels stream each 16-token chunk of K and
 * V once for all query heads of its kv-head.
 *
 *   out  [num_seqs, num_heads, head_dim]  (written)
 *   q    [num_seqs, num_heads, head_dim]
 *   out[b][h] = softmax_j(scale * q[b][h] . K_b[j] (+ mods)) V_b[j], j < context_lens[b]
 *
 * max_context_len is a host-side upper bound of context_lens that sizes the
 * launch (no device->host sync); larger device values are undefined
 * behaviour.  scale is any finite value (usually 1/sqrt(head_dim); 0 weights
 * every key alike).  A sequence with context_len 0 gets a zero output.  The
 * workspace (device memory of at least
 * paged_attn_decode_workspace_size(...) bytes; may be NULL when that size is
 * 0) holds per-partition partial results between the two kernels.
 * Equivalent to paged_attn_decode_partials followed by
 * paged_attn_decode_merge with the same arguments.
 */
int paged_attn_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, int32_t block_table_stride,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                      int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                      int64_t num_blocks, int32_t max_context_len, float scale,
                      int32_t split_tokens, const pa_score_mods* mods, void* workspace,
                      size_t workspace_bytes, int32_t dtype, void* stream);

/*
 * paged_attn_decode_noalloc -- paged_attn_decode with no workspace argument,
 * for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops that must not call hipMalloc, harnesses that forbid
 * it.  Arguments, result and status codes as paged_attn_decode.
 *
 * The partial results live in a scratch array the library holds on each
 * device (PA_DECODE_SCRATCH_BYTES = 16 MiB, allocated with the library's
 * code on that device and kept until the process ends).  A call whose
 * workspace would exceed it -- paged_attn_decode_workspace_size() of the
 * same sizes above PA_DECODE_SCRATCH_BYTES -- returns PA_ERR_SCRATCH and
 * enqueues nothing (the long-context batch of 64 sequences x 8 kv-heads x
 * 8 query heads per kv-head, D 128, needs 10.6 MB).  The call allocates
 * nothing: no hipMalloc, no hipFree, no library routine that allocates.
 * Every call on a device shares that device's array and leaves its contents
 * behind; each call writes everything it reads there before reading it.
 * Calls that overlap on one device (two streams, two threads) race on the
 * array and give undefined results: order them on one stream, or use
 * paged_attn_decode with workspaces of your own.
 */
#define PA_DECODE_SCRATCH_BYTES (16u << 20)

int paged_attn_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, int32_t num_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                              int64_t num_blocks, int32_t max_context_len, float scale,
                              int32_t split_tokens, const pa_score_mods* mods, int32_t dtype,
                              void* stream);

/*
 * The two phases of paged_attn_decode as separate calls (same arguments).
 * _partials runs the partition kernel: sequences whose context fits one
 * partition get their final output; the others leave unnormalised partial
 * outputs with their running max and sum in the workspace.  _merge combines
 * those partials (log-sum-exp weighting, fixed partition order) into out and
 * launches nothing when no sequence can span more than one partition.
 */
int paged_attn_decode_partials(void* out, const void* q, const void* k_cache,
                               const void* v_cache, const int32_t* block_tables,
                               int32_t block_table_stride, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int64_t num_blocks,
                               int32_t max_context_len, float scale, int32_t split_tokens,
                               const pa_score_mods* mods, void* workspace,
                               size_t workspace_bytes, int32_t dtype, void* stream);

int paged_attn_decode_merge(void* out, const int32_t* context_lens, int32_t num_seqs,
                            int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t max_context_len, int32_t split_tokens,
                            const pa_score_mods* mods, const void* workspace,
                            size_t workspace_bytes, int32_t dtype, void* stream);

/*
 * Two-phase decode for sequences that share a prefix.
 *
 * Requests that start with the same prompt share the prefix's physical
 * blocks ("Ultimate Guide to PagedAttention": block table and scheduler,
 * memory sharing), so a decode step over such a batch reads the same keys once
 * per sequence.  This call instead computes each shared part once per group
 * of sharing sequences, with all the group's query rows against those keys on
 * the matrix cores, then each sequence's own keys with the paged decode, and
 * combines the softmax states by their log-sum-exps -- the prefix-first, then
 * sequence-first split that the related-paper list of "Paged Attention Meets
 * FlexAttention" (fugumt.com) describes for ChunkAttention.  Shared parts may
 * be nested (a system prompt shared by all, then a conversation shared by its
 * beams: the hierarchical prefixes the vAttention page's decode snippets
 * speak of), one level per nesting depth.  The result is the same attention
 * as paged_attn_decode (up to rounding order; the shared parts' softmax
 * weights are rounded to bf16 before the P.V product, as in
 * paged_attn_prefill).
 *
 * One pa_prefix_level per depth, levels[0] outermost.  At every level the
 * groups partition the batch into runs of consecutive sequences:
 *   group_starts  device int32 [num_groups + 1]: sequences group_starts[g] ..
 *                 group_starts[g+1]-1 form group g; group_starts[0] = 0,
 *                 non-decreasing, group_starts[num_groups] = num_seqs (a
 *                 group may have one member or none).
 *   prefix_starts device int32 [num_groups], or NULL for all 0;
 *   prefix_ends   device int32 [num_groups]: group g shares keys
 *                 [prefix_starts[g], prefix_ends[g]) -- the same key/value
 *                 vectors for every member, read through the table row of
 *                 the group's first member.
 *   num_groups (>= 1), max_group_size (host bound on members per group,
 *   >= 1), max_prefix_len (host bound on prefix_ends[g] - prefix_starts[g]).
 * For every sequence the ranges of its groups must follow each other: level
 * 0 starts at key 0, level l + 1 starts where level l ended, and the last end
 * is at most the sequence's context length; its own keys are the rest.  An
 * empty range (start == end) is allowed.  1 <= num_levels <= 8.
 *
 * Other arguments, score mods included, as paged_attn_decode (the shared
 * parts see each row at its own sequence's position for the window and
 * ALiBi, and its document start).  bf16 only, num_heads / num_kv_heads must
 * divide 128.  The workspace is device memory of at least
 * paged_attn_decode_cascade_workspace_size(...) bytes, 16-byte aligned (the
 * size function reads only the levels' host fields).  Breaking the
 * device-side contract (groups, ranges) is undefined behaviour; the debug
 * library traps.
 *
 * paged_attn_decode_cascade picks the faster of the two-phase decode and the
 * plain paged_attn_decode for the batch: below 256 MiB of logical K+V
 * (num_seqs x max_context_len keys, K and V, every kv-head: the host-side
 * bound) a decode step is bound by launches rather than by re-reading the
 * shared keys, and the plain decode (run in the same workspace) is faster;
 * paged_attn_decode_cascade_plan() tells which one a call will run (1:
 * two-phase, 0: plain).  paged_attn_decode_cascade_two_phase always runs the
 * two-phase decode.  Both give the same attention up to rounding order.
 */
typedef struct {
  const int32_t* group_starts;
  const int32_t* prefix_starts;
  const int32_t* prefix_ends;
  int32_t num_groups;
  int32_t max_group_size;
  int32_t max_prefix_len;
} pa_prefix_level;

size_t paged_attn_decode_cascade_workspace_size(int32_t num_seqs, const pa_prefix_level* levels,
                                                int32_t num_levels, int32_t num_heads, int32_t num_kv_heads,
                                                int32_t head_dim, int32_t max_context_len);

int paged_attn_decode_cascade(void* out, const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t block_table_stride,
                              const int32_t* context_lens, int32_t num_seqs, const pa_prefix_level* levels,
                              int32_t num_levels, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                              int32_t block_size, int64_t num_blocks, int32_t max_context_len, float scale,
                              const pa_score_mods* mods, void* workspace, size_t workspace_bytes, int32_t dtype,
                              void* stream);

int paged_attn_decode_cascade_two_phase(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t block_table_stride,
                                        const int32_t* context_lens, int32_t num_seqs,
                                        const pa_prefix_level* levels, int32_t num_levels, int32_t num_heads,
                                        int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                                        int64_t num_blocks, int32_t max_context_len, float scale,
                                        const pa_score_mods* mods, void* workspace, size_t workspace_bytes,
                                        int32_t dtype, void* stream);

/* 1 if paged_attn_decode_cascade would run the two-phase decode for these
 * sizes, 0 if the plain decode (or invalid arguments). */
int32_t paged_attn_decode_cascade_plan(int32_t num_seqs, const pa_prefix_level* levels, int32_t num_levels,
                                       int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                       int32_t max_context_len);

/*
 * paged_attn_prefill -- several query rows per sequence (prefill, or a
 * chunk appended after an existing paged context) over the paged context.
 *
 * The fused kernel gathers each key tile from the scattered blocks straight
 * into on-chip memory and never forms a contiguous copy (Joshi et al.,
 * "Paged Attention Meets FlexAttention", abstract: a fused kernel that
 * gathers scattered KV data), computing exact attention tile by tile with an
 * online softmax (Dao et al., "FlashAttention", abstract: IO-aware tiling for
 * exact attention).
 *
 *   q, out  [total_q, num_heads, head_dim]; sequence b owns rows
 *           cu_q_lens[b] .. cu_q_lens[b+1]-1 (cu_q_lens: int32 [num_seqs+1],
 *           device), its L = cu_q_lens[b+1]-cu_q_lens[b] rows sit at logical
 *           positions context_lens[b]-L .. context_lens[b]-1.
 *   causal  1: a row sees keys at positions <= its own; 0: all keys.
 *   max_q_len: host-side upper bound of the per-sequence row counts.
 *   scale   any finite value, as for the decode.
 *
 * The chunk's own keys/values must already be in the cache (kv_append first),
 * so a row always sees itself.  bf16 runs on matrix cores (bf16 products, fp32
 * accumulation, softmax weights rounded to bf16 before the P.V product); fp32
 * runs on vector ALUs in fp32.  Rows with no admissible key are zero.
 */
int paged_attn_prefill(void* out, const void* q, const int32_t* cu_q_lens, const void* k_cache,
                       const void* v_cache, const int32_t* block_tables,
                       int32_t block_table_stride, const int32_t* context_lens,
                       int32_t num_seqs, int32_t max_q_len, int32_t num_heads,
                       int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                       int64_t num_blocks, float scale, int32_t causal,
                       const pa_score_mods* mods, int32_t dtype, void* stream);

/*
 * paged_attn_prefill_split -- paged_attn_prefill whose key range may be split
 * over several work-groups per query tile, for grids of (sequence, kv-head,
 * query tile) too small to fill the device (one GPU's share of a split over
 * heads, short chunks of few sequences).  Each range computes exact
 * attention over its keys as a normalised output and its log-sum-exp; a
 * merge weights them by those exponentials, which gives the same softmax
 * over the whole range (Dao et al., "FlashAttention", abstract: exact
 * attention from tiles; the decode's split partitions are merged the same
 * way).
 *
 *   total_q          rows of q and out (= cu_q_lens[num_seqs]; a different
 *                    value is undefined behaviour, checked in debug builds)
 *   max_context_len  host-side upper bound of context_lens (as for the
 *                    decode; it sizes the key ranges)
 *   key_split        0: the library's choice (a bf16 grid with fewer
 *                    work-groups than compute units gets ranges of at least
 *                    512 keys, up to about two work-groups per unit);
 *                    -1: never split; > 0: keys per range, a multiple of 64
 *                    (PA_ERR_SPLIT otherwise)
 *   workspace        device memory of at least
 *                    paged_attn_prefill_workspace_size(...) bytes (fp32 range
 *                    states; may be NULL when that size is 0)
 *
 * Other arguments, masks and score mods as paged_attn_prefill.  Without a
 * split (fp32, a grid that fills the device, key_split -1, a single range, or
 * a block mask) the call is exactly paged_attn_prefill and ignores the
 * workspace.  Otherwise the rounding order differs from the unsplit call
 * (fp32 range states, bf16 output once at the end).  Returns PA_ERR_WORKSPACE
 * when a split needs more workspace than given, PA_ERR_SIZE when total_q or
 * max_context_len is negative or the sizes overflow.
 */
size_t paged_attn_prefill_workspace_size(int32_t num_seqs, int32_t total_q, int32_t max_q_len,
                                         int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                                         int32_t max_context_len, int32_t key_split, int32_t dtype);
int paged_attn_prefill_split(void* out, const void* q, const int32_t* cu_q_lens, int32_t total_q,
                             const void* k_cache, const void* v_cache, const int32_t* block_tables,
                             int32_t block_table_stride, const int32_t* context_lens, int32_t num_seqs,
                             int32_t max_q_len, int32_t num_heads, int32_t num_kv_heads, int32_t head_dim,
                             int32_t block_size, int64_t num_blocks, int32_t max_context_len,
                             int32_t key_split, float scale, int32_t causal, const pa_score_mods* mods,
                             void* workspace, size_t workspace_bytes, int32_t dtype, void* stream);

/* Human-readable name of a status code (static string). */
const char* paged_attn_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
