/*
 * paged_block_manager.h -- host-side manager of the physical KV blocks behind
 * the block tables that paged_attn_decode consumes (C ABI).
 *
 * The pool holds num_blocks physical blocks of block_size tokens. The manager
 * keeps what page "paged-attention-runtime" (design notes, BlockManager) lists:
 * a free list, a reference count per block, and each sequence's list of block
 * ids, with the operations allocate_blocks, free_sequence, share_prefix (a
 * target sequence starts with a source's first blocks, whose reference counts
 * rise) and cow_block (copy-on-write: a shared block a sequence is about to
 * modify is replaced by a fresh one); a block returns to the free list when its
 * reference count reaches zero. On top of those: the block table of a batch in
 * the layout paged_attn_decode reads, and append_slot, the bookkeeping of a
 * decode step that writes token seq_len of a sequence.
 *
 * Host memory only; the manager never touches the device. Copy-on-write
 * returns the (source, destination) block pair whose K/V contents the caller
 * copies, e.g. with paged_attn_copy_blocks. Ids are handed out lowest first, so
 * a sequence of operations gives the same tables every time. Not thread-safe:
 * one manager is used by one thread at a time. Errors are the PA_E_* codes of
 * paged_attn.h; an operation that fails changes nothing.
 */
#ifndef PAGED_BLOCK_MANAGER_H
#define PAGED_BLOCK_MANAGER_H

#include <stddef.h>
#include <stdint.h>

#include "paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_block_manager pa_block_manager; /* opaque */

/* A manager of blocks 0 .. num_blocks-1, all free. NULL if num_blocks <= 0,
 * block_size is not a power of two in [1, 1024], or memory runs out. */
pa_block_manager* paged_attn_bm_create(int32_t num_blocks, int32_t block_size);
/* Frees the manager (NULL is ignored). */
void paged_attn_bm_destroy(pa_block_manager* bm);

/* Appends n fresh blocks (reference count 1) to sequence seq_id, creating the
 * sequence if it has none. PA_E_NOMEM if fewer than n blocks are free,
 * PA_E_SHAPE if n < 0, PA_E_NULL for a NULL manager. */
int paged_attn_bm_allocate_blocks(pa_block_manager* bm, int64_t seq_id, int32_t n);
/* Drops sequence seq_id: each of its blocks loses one reference and returns to
 * the free list at zero. PA_E_SEQ if the sequence is unknown. */
int paged_attn_bm_free_sequence(pa_block_manager* bm, int64_t seq_id);
/* Starts sequence `target` (which must not exist yet) with the first n_blocks
 * blocks of `source`, each gaining one reference. PA_E_SEQ if source is unknown,
 * holds fewer than n_blocks blocks, or target exists; PA_E_SHAPE if n_blocks < 0. */
int paged_attn_bm_share_prefix(pa_block_manager* bm, int64_t source, int64_t target,
                               int32_t n_blocks);
/* Makes block block_index of seq_id exclusive to it. Returns 0 when it already
 * was (nothing changes), 1 when a fresh block replaced it: *src is the old
 * (still shared) block, *dst the new one, whose K/V the caller must fill from
 * *src before the sequence's next read. PA_E_SEQ for an unknown sequence or
 * index, PA_E_NOMEM when no block is free. */
int paged_attn_bm_cow_block(pa_block_manager* bm, int64_t seq_id, int32_t block_index,
                            int32_t* src, int32_t* dst);
/* Readies the slot of token seq_len (0-based) of seq_id for a write: allocates a
 * block when the token starts a new one, and copy-on-writes the token's block
 * when it is shared. seq_id may be new when seq_len == 0. Returns 0, or 1 with
 * the copy to make in *src / *dst as for cow_block. PA_E_SEQ if the sequence
 * holds fewer than seq_len / block_size blocks (a gap) or seq_len < 0,
 * PA_E_NOMEM when no block is free. */
int paged_attn_bm_append_slot(pa_block_manager* bm, int64_t seq_id, int32_t seq_len,
                              int32_t* src, int32_t* dst);

/* Number of free blocks, or PA_E_NULL. */
int paged_attn_bm_num_free(const pa_block_manager* bm);
/* Reference count of a block (0 when free), or PA_E_SEQ if out of range. */
int paged_attn_bm_ref_count(const pa_block_manager* bm, int32_t block);
/* Copies up to `cap` of seq_id's block ids into out (may be NULL when cap is 0)
 * and returns how many blocks it holds, or PA_E_SEQ if unknown. */
int paged_attn_bm_sequence_blocks(const pa_block_manager* bm, int64_t seq_id, int32_t* out,
                                  int32_t cap);
/* Fills table [batch, max_blocks_per_seq] (row-major, host memory) with the
 * block ids of seq_ids[0 .. batch-1], padded with -1: the block_table argument
 * of paged_attn_decode. PA_E_SEQ if a sequence is unknown, PA_E_SHAPE if one
 * holds more than max_blocks_per_seq blocks. */
int paged_attn_bm_block_table(const pa_block_manager* bm, const int64_t* seq_ids, int32_t batch,
                              int32_t max_blocks_per_seq, int32_t* table);

/* Device side of copy-on-write: for each of the n pairs (src, dst) in `pairs`
 * (device int32 [n, 2]), copies every KV head's block_size token rows of block
 * src into block dst, in both k_cache and v_cache (pools described by desc).
 * Enqueued on `stream`; a pair with an id outside [0, num_blocks) is skipped
 * and sets PA_STATUS_BAD_BLOCK in the optional device status word. Returns
 * PA_OK, a descriptor error, PA_E_NULL or PA_E_LAUNCH. Pairs must not chain
 * (no dst is another pair's src). */
int paged_attn_copy_blocks(const pa_desc* desc, void* k_cache, void* v_cache, const int32_t* pairs,
                           int32_t n, int32_t* status, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGED_BLOCK_MANAGER_H */
