/*
 * pkv_block_manager.h -- host-side block manager of libpagedkv.so: the
 * allocator that hands out the physical blocks of a paged KV pool and keeps
 * the per-sequence block tables the kernels of pagedkv.h read.
 *
 * What it does, after the pages:
 *   [P2 sec. 2.1] a global pool of fixed-size physical blocks; per-sequence
 *     block tables (logical block i -> physical id); allocate, free,
 *     append_slot (the decode step's new token: the next slot of the last
 *     block if it has room, else a new block) and can_allocate.
 *   [P3 sec. 2.2] a table holds its block ids in logical order and the
 *     first-block offset; capacity = blocks * block_size - offset.
 *   [P3 sec. 2.3] allocation needs ceil((offset + tokens) / block_size)
 *     blocks and takes them one by one from the front of a FIFO queue of
 *     free ids; when the queue is short the answer is "no" and nothing is
 *     taken (PKV_NO_SPACE here).
 *   [P3 sec. 2.4] reference counts: a block shared by several tables goes
 *     back to the free queue (at its back) only when its count reaches 0.
 *   [P3 sec. 3.1] copy-on-write: a sequence about to write into a shared
 *     block first gets a private copy (pkv_bm_cow, then kv_copy_blocks).
 *
 * Sequences are named by caller-chosen int64 ids.  A manager is plain host
 * memory; calls on one manager must not overlap (it has no lock).  All
 * entry points return a status of pagedkv.h (PKV_OK, PKV_NO_SPACE or a
 * negative error) unless stated otherwise; on an error nothing changes.
 */
#ifndef PKV_BLOCK_MANAGER_H
#define PKV_BLOCK_MANAGER_H

#include "pagedkv.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkv_block_manager pkv_block_manager;

typedef struct pkv_bm_stats {
    int64_t num_blocks;
    int64_t block_size;
    int64_t free_blocks;       /* length of the free queue                    */
    int64_t used_blocks;       /* num_blocks - free_blocks                    */
    int64_t peak_used_blocks;  /* largest used_blocks since creation          */
    int64_t live_tokens;       /* distinct (block, slot) pairs holding a token */
    int64_t num_seqs;
} pkv_bm_stats;

/* A manager of num_blocks blocks of block_size slots, all free, queued in
 * id order 0 .. num_blocks-1.  NULL for sizes <= 0 or when host memory runs
 * out.  Release with pkv_bm_destroy. */
PKV_API pkv_block_manager *pkv_bm_create(int32_t num_blocks, int32_t block_size);
PKV_API void pkv_bm_destroy(pkv_block_manager *bm);

/* 1 if a sequence of num_tokens tokens starting at `offset` in its first
 * block could be allocated now, 0 if not, < 0 for bad arguments. */
PKV_API int pkv_bm_can_allocate(const pkv_block_manager *bm, int64_t num_tokens, int32_t offset);

/* New sequence `seq` holding num_tokens tokens from flat position `offset`
 * (0 <= offset < block_size) of its table [P3 sec. 2.3].  PKV_NO_SPACE when
 * the free queue is short.  Errors: PKV_ERR_NULL, _SHAPE, _SEQ (exists). */
PKV_API int pkv_bm_allocate(pkv_block_manager *bm, int64_t seq, int64_t num_tokens, int32_t offset);

/* New sequence `dst` whose table starts with the first num_blocks blocks of
 * `src` (one more reference each [P3 sec. 2.4]) and src's offset; it holds
 * num_blocks*block_size - offset tokens (whole-block prefix sharing).
 * Errors: PKV_ERR_NULL, _SHAPE (num_blocks outside [1, src's blocks]), _SEQ. */
PKV_API int pkv_bm_share(pkv_block_manager *bm, int64_t src, int64_t dst, int32_t num_blocks);

/* One more token for `seq` [P2 sec. 2.1]: *slot receives its slot
 * (block * block_size + position in block), taking a new block from the
 * free queue when the last one is full.  PKV_NO_SPACE (nothing changed)
 * when that block is not there.  Errors: PKV_ERR_NULL, _SEQ. */
PKV_API int pkv_bm_append_slot(pkv_block_manager *bm, int64_t seq, int64_t *slot);

/* pkv_bm_append_slot for seqs[0..n) in order, slots[i] for each.  Returns
 * how many were appended: n when all, fewer when one met PKV_NO_SPACE or
 * host memory ran out (the rest untouched); or a negative error from the
 * argument checks, made before any append (then nothing changed). */
PKV_API int32_t pkv_bm_append_slots(pkv_block_manager *bm, const int64_t *seqs, int32_t n,
                                    int64_t *slots);

/* Drop `seq`: one reference less for each of its blocks, in table order;
 * blocks whose count reaches 0 join the back of the free queue.
 * Errors: PKV_ERR_NULL, _SEQ. */
PKV_API int pkv_bm_free(pkv_block_manager *bm, int64_t seq);

/* Copy-on-write of table entry `index` of `seq` [P3 sec. 3.1: sharing by
 * copy-on-write + ref_count], before the sequence writes into that block.
 * When the block has other holders (count > 1), the free queue's front
 * block takes its place in this table (count 1, as in allocate
 * [P3 sec. 2.3]) and the old block loses one reference [P3 sec. 2.4];
 * *src_block / *dst_block receive old and new: copy its contents with
 * kv_copy_blocks.  An unshared block needs no copy: both receive it and
 * nothing changes.  PKV_NO_SPACE (nothing changed) when a copy is needed
 * and no block is free.  Errors: PKV_ERR_NULL, _SEQ, _SHAPE (index outside
 * the table). */
PKV_API int pkv_bm_cow(pkv_block_manager *bm, int64_t seq, int32_t index, int32_t *src_block,
                       int32_t *dst_block);

/* One more / one less holder of a used block [P3 sec. 2.4]; dec_ref to 0
 * frees it.  Errors: PKV_ERR_NULL, _BLOCK (out of range or free). */
PKV_API int pkv_bm_inc_ref(pkv_block_manager *bm, int32_t block);
PKV_API int pkv_bm_dec_ref(pkv_block_manager *bm, int32_t block);

/* Tokens held by `seq` (< 0: PKV_ERR_NULL or PKV_ERR_SEQ). */
PKV_API int64_t pkv_bm_seq_len(const pkv_block_manager *bm, int64_t seq);

/* Most blocks in the tables of seqs[0..n): the bt_stride pkv_bm_tables
 * needs (< 0 on error). */
PKV_API int32_t pkv_bm_max_blocks(const pkv_block_manager *bm, const int64_t *seqs, int32_t n);

/* The kernels' inputs for seqs[0..n), in host memory: tables (n, stride)
 * row-major, padded with -1; seq_lens and offsets [n] (either may be NULL).
 * Errors: PKV_ERR_NULL, _SHAPE (a table longer than stride), _SEQ. */
PKV_API int pkv_bm_tables(const pkv_block_manager *bm, const int64_t *seqs, int32_t n,
                          int32_t *tables, int32_t stride, int32_t *seq_lens, int32_t *offsets);

/* The free queue front to back, up to cap ids; returns its full length. */
PKV_API int32_t pkv_bm_free_queue(const pkv_block_manager *bm, int32_t *ids, int32_t cap);

/* Reference counts of blocks 0 .. min(cap, num_blocks)-1; returns num_blocks. */
PKV_API int32_t pkv_bm_ref_counts(const pkv_block_manager *bm, int32_t *counts, int32_t cap);

PKV_API int pkv_bm_get_stats(const pkv_block_manager *bm, pkv_bm_stats *out);

#ifdef __cplusplus
}
#endif

#endif /* PKV_BLOCK_MANAGER_H */
