/*
 * pagedattn_blocks.h -- host-side block manager for the paged KV cache.
 *
 * The pool of physical blocks is handed out to sequences on demand; a
 * sequence's block table maps its logical blocks to physical ones, sequences
 * that share a prefix (a forked beam, a common prompt) share physical blocks
 * through reference counts, and a write into a shared, partially filled block
 * first copies it (copy-on-write) ("Ultimate Guide to PagedAttention":
 * block table, dynamic allocation, memory sharing and copy-on-write; Kwon et
 * al., "Efficient Memory Management for Large Language Model Serving with
 * PagedAttention", abstract: near-zero waste and flexible sharing).
 *
 * Pages are aligned runs of 1, 2, 4, ... consecutive blocks, handed out by a
 * buddy allocator (split on demand, merged with a free buddy on release).  A
 * sequence's pages have one size, or double along the sequence up to a cap:
 * power-of-two cache growth, as in "Paged Attention Meets FlexAttention"
 * (abstract: memory grows at power-of-two allocation steps).  One pool can
 * hold sequences with different page sizes.  Block tables stay at block
 * resolution (a page of 2^k blocks is 2^k consecutive entries), so the
 * attention calls read a mixed pool as an ordinary pool of block_size-token
 * blocks; pa_bm_create / pa_bm_new_sequence are the one-block-page case.
 *
 * This is bookkeeping on the host only: it produces the slot_mapping that
 * kv_append consumes, the block-table rows the attention calls read, and the
 * (src, dst) block pairs that kv_copy_blocks must copy before the append.
 * It never touches device memory.  Every call is thread-safe (one lock per
 * manager).  Status codes are those of pagedattn.h; the manager adds
 * PA_ERR_NO_BLOCKS (the pool is exhausted; the call changed nothing) and
 * PA_ERR_SEQ (unknown or freed sequence id).
 */
#ifndef PAGEDATTN_BLOCKS_H_
#define PAGEDATTN_BLOCKS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager;

/* A manager for num_blocks physical blocks of block_size tokens (a power of
 * two in [16, 256]), with pages of one block.  Slots are int32, so
 * num_blocks * block_size must stay below 2^31 (else PA_ERR_SIZE).  *out
 * receives the handle; NULL on failure. */
int pa_bm_create(int64_t num_blocks, int32_t block_size, pa_block_manager** out);

/* The same with pages of up to max_page_blocks blocks (a power of two,
 * 1..4096).  The pool starts as aligned free pages as large as alignment and
 * num_blocks allow.  PA_ERR_SIZE for a max_page_blocks out of range. */
int pa_bm_create_paged(int64_t num_blocks, int32_t block_size, int32_t max_page_blocks, pa_block_manager** out);
void pa_bm_destroy(pa_block_manager* bm);

/* A new, empty sequence with one-block pages; its id goes to *seq. */
int pa_bm_new_sequence(pa_block_manager* bm, int32_t* seq);

/* A new, empty sequence whose page k (k = 0, 1, ...) has
 * min(min_page_blocks << k, max_page_blocks) blocks: equal bounds give one
 * page size, different bounds pages that double along the sequence.  Both
 * are powers of two with min_page_blocks <= max_page_blocks <= the manager's
 * max_page_blocks (else PA_ERR_SIZE).  If the pool has no free page of the
 * size due, the largest smaller free page stands in.  Forks keep the
 * parent's pages and rule. */
int pa_bm_new_sequence_paged(pa_block_manager* bm, int32_t min_page_blocks, int32_t max_page_blocks, int32_t* seq);

/* A new sequence that shares every page (and the length) of `parent`
 * (reference counts rise; nothing is copied yet). */
int pa_bm_fork(pa_block_manager* bm, int32_t parent, int32_t* child);

/* Drop a sequence; pages whose count falls to zero return to the pool. */
int pa_bm_free_sequence(pa_block_manager* bm, int32_t seq);

/*
 * Reserve slots for ntok new tokens at the end of `seq`, taking new pages
 * as needed.  slots_out[i] (ntok entries) is the pool slot of logical
 * position len + i, as kv_append expects.  If the last page is shared and
 * has free slots (other owners would write into the same slots), it is
 * first replaced by a fresh page of the same size, and the (old, new) pairs
 * of its blocks that hold tokens go to copy_src/copy_dst (room for copy_cap
 * pairs, at most the page's block count; *ncopy receives the count): the
 * caller runs kv_copy_blocks on those pairs before kv_append.
 * PA_ERR_NO_BLOCKS leaves everything unchanged; PA_ERR_SIZE if ntok < 0 or
 * copy_cap is too small.
 */
int pa_bm_append(pa_block_manager* bm, int32_t seq, int32_t ntok, int32_t* slots_out,
                 int32_t* copy_src, int32_t* copy_dst, int32_t copy_cap, int32_t* ncopy);

/* The sequence's token count (*len) and block-table row: the first
 * min(cap, nblocks) entries go to row, the total to *nblocks. */
int pa_bm_table(const pa_block_manager* bm, int32_t seq, int32_t* row, int32_t cap, int32_t* nblocks,
                int64_t* len);

/* Pool accounting: free blocks, blocks in use, and the slots of blocks in
 * use that hold no token (internal fragmentation = waste / (used * bs)). */
int pa_bm_stats(const pa_block_manager* bm, int64_t* free_blocks, int64_t* used_blocks, int64_t* waste_slots);

/* The sequence's pages in order: first block (starts) and size in blocks
 * (blocks) of the first min(cap, npages) pages; the total goes to *npages. */
int pa_bm_pages(const pa_block_manager* bm, int32_t seq, int32_t* starts, int32_t* blocks, int32_t cap,
                int32_t* npages);

/* Reference count of one physical block (0 = free; equal over a page). */
int pa_bm_block_refcount(const pa_block_manager* bm, int32_t block, int32_t* count);

/*
 * Shared prefixes of a decode batch, as the levels paged_attn_decode_cascade
 * takes (pagedattn.h).  seqs[0..n) is the batch in the caller's order (put
 * sequences forked from one another next to each other: only neighbours in
 * this order are grouped).  Two neighbours share the leading full blocks
 * that both tables name identically (blocks shared by fork; a partly filled
 * block is never counted).  Level 0 groups maximal runs of neighbours that
 * share at least one block, with the run's common part as range [0, end);
 * each deeper level splits every group the same way over what its members
 * share beyond the previous end.  A sequence left alone, or a run that shares
 * nothing more, continues as a group with an empty range, so every level
 * partitions the batch and ranges chain.
 *
 * Host output arrays, one row per level (at most max_levels, 1..8):
 * group_starts [max_levels][n + 1], prefix_starts and prefix_ends
 * [max_levels][n], num_groups [max_levels]; *num_levels gets the levels
 * used -- 0 when no two neighbours share a block (then the plain decode is
 * the right call).  Sharing deeper than max_levels stays in the sequences'
 * own keys (still correct, computed per sequence).  PA_ERR_SEQ for an
 * unknown id, PA_ERR_SIZE for n < 0 or max_levels outside 1..8.
 */
int pa_bm_prefix_levels(const pa_block_manager* bm, const int32_t* seqs, int32_t n, int32_t max_levels,
                        int32_t* group_starts, int32_t* prefix_starts, int32_t* prefix_ends, int32_t* num_groups,
                        int32_t* num_levels);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_BLOCKS_H_ */
