/*
 * pagedkv.h -- C ABI of the MI355X (gfx950) paged KV-cache library
 * (libpagedkv.so).
 *
 * The library implements block-table-indirected access to a paged KV cache:
 * the slot computation, the slot_mapping scatter of new K/V rows into the
 * pool, the block_table gather into contiguous K/V, and fused paged decode
 * attention that reads the scattered blocks in place.
 *
 * Sources (three web pages on paged KV caches):
 *   [P1] mini-vllm tutorial, "step14_2 - index_select gather"
 *   [P2] "vLLM PagedAttention source notes" (minivLLM Task 6 background)
 *   [P3] mini-runtime, chapter 12 "Paged KV Cache"
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Pool layout [P2 sec. 2.2]: K and V are separate, each a contiguous
 *   (num_blocks, num_layers, block_size, num_kv_heads, head_dim) array in
 *   device memory.  One "row" is the num_kv_heads*head_dim elements of one
 *   token at one layer.  block_size must be a power of two.
 * - Element types: PKV_F32 (float) or PKV_BF16 (bfloat16 bit patterns),
 *   or a quantised pool, PKV_I8 or PKV_I4 (see "Quantised pools" below).
 * - A block table is a row of int32 physical block ids in logical order
 *   [P3 sec. 2.2]; tables are stored (num_seqs, bt_stride) row-major.  Each
 *   sequence also has a first-block start offset in [0, block_size) (prefix
 *   sharing creates it [P3 sec. 2.2]): logical token t of the sequence sits
 *   at flat position offset + t of its table, i.e. in block
 *   table[(offset+t) / block_size] at slot (offset+t) % block_size.
 *   A table holds len*block_size - offset tokens [P3 sec. 2.2].
 * - Pointers named "device" are device memory owned by the caller; the
 *   library allocates and frees nothing, keeps no per-call state and never
 *   synchronises (except where stated).  All work is enqueued on `stream`
 *   (a hipStream_t; NULL = the default stream); the return value covers
 *   argument checks and the launch only.
 * - Every base pointer that the kernels read or write in 16-byte pieces
 *   (pools, q, K/V sources and outputs, workspace) must be 16-byte aligned,
 *   and a row (num_kv_heads*head_dim*element size) must be a multiple of 16
 *   bytes; otherwise PKV_ERR_ALIGN.
 * - Arguments are checked on the host before any HIP call; a failed check
 *   returns a negative status and enqueues nothing.  No exception or abort
 *   crosses this ABI.
 * - Device-resident ids are not range-checked by the fast entry points'
 *   contract.  For safety the kernels still never touch memory outside the
 *   pool, the tables or the outputs: a slot or block id that is out of range
 *   is treated as padding (scatter skips the row, gather writes a zero row,
 *   decode masks the token).  kv_validate counts such violations.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PKV_API __attribute__((visibility("default")))

/* element types */
enum { PKV_F32 = 0, PKV_BF16 = 1, PKV_I8 = 2, PKV_I4 = 3 };

/* status codes */
enum {
    PKV_OK = 0,
    PKV_ERR_NULL = -1,        /* a required pointer is NULL                    */
    PKV_ERR_DTYPE = -2,       /* unknown element type                          */
    PKV_ERR_SHAPE = -3,       /* negative/zero size, non power-of-two block    */
                              /* size, num_q_heads % num_kv_heads != 0, ...    */
    PKV_ERR_LAYER = -4,       /* layer outside [0, num_layers)                 */
    PKV_ERR_ALIGN = -5,       /* pointer or row not 16-byte aligned            */
    PKV_ERR_WORKSPACE = -6,   /* workspace missing or smaller than required    */
    PKV_ERR_LAUNCH = -7,      /* the HIP launch reported an error              */
    PKV_ERR_UNSUPPORTED = -8, /* head_dim / query-group size not compiled in   */
    PKV_ERR_DEVICE = -9,      /* no usable HIP device                          */
    PKV_ERR_SEQ = -10,        /* block manager: unknown or duplicate sequence  */
    PKV_ERR_BLOCK = -11,      /* block manager: block id out of range or free  */
    PKV_ERR_HOST = -12,       /* host memory could not be allocated            */
    PKV_ERR_SCRATCH = -13,    /* paged_attn_decode_noalloc: the sizes need     */
                              /* more than PKV_NOALLOC_SCRATCH_BYTES           */
    PKV_NO_SPACE = 1          /* block manager: too few free blocks; nothing   */
                              /* was changed (not an error)                    */
};

/* A paged KV pool: caller-owned device memory, only read or written during
 * a call.  dtype is PKV_F32 or PKV_BF16; `reserved` must be 0.  K and V are
 * each laid out as (num_blocks, num_layers, block_size, num_kv_heads,
 * head_dim) [P2 sec. 2.2]; block_stride is the byte distance from one block
 * of a tensor to the next, 0 meaning the dense layout (num_layers *
 * block_size * num_kv_heads * head_dim * element bytes).  The combined
 * layout (num_blocks, 2, num_layers, block_size, num_kv_heads, head_dim)
 * of the same section is k = its base, v = base + one dense block,
 * block_stride = two dense blocks.  A nonzero block_stride must be a
 * multiple of 16 and at least one dense block.
 *
 * Quantised pools (dtype PKV_I8, PKV_I4) [P3 sec. 6: quantised KV, int8 / int4, as
 * the next compression step of a paged cache; the pages give no method, so
 * this is the plain symmetric reading]: k / v hold int8 codes in the layout
 * above, and k_scale / v_scale (16-byte aligned, device) one float scale
 * per (token, kv head) row, laid out dense as
 * (num_blocks, num_layers, num_kv_heads, block_size), so the scales of one
 * head's tokens in a block are contiguous.  A row x (head_dim values) is
 * stored as scale s = max|x| / 127 and codes round-half-even(x / s),
 * clamped to [-127, 127] (s = 0 and codes 0 for a zero row), both
 * computed in IEEE float32; its value is code * s.  PKV_I4 is the same
 * reading at four bits: s = max|x| / 7, codes in [-7, 7], two codes per
 * byte -- element 2i of a row in the low nibble of byte i, element 2i + 1
 * in the high nibble, four-bit two's complement -- so a row is
 * num_kv_heads * head_dim / 2 bytes in the layout above.  The rows written
 * into (k_src / v_src) and the queries and outputs of decode are bfloat16.
 * Entry points that take a quantised pool: kv_scatter, kv_append
 * (quantise on write), kv_gather (writes bf16(code * s)),
 * paged_attn_decode (split and planned schedules; dequantises inside the
 * kernel), kv_copy_blocks and kv_swap_out / kv_swap_in (codes and
 * scales).  The others return PKV_ERR_UNSUPPORTED for it.  k_scale /
 * v_scale are ignored for float pools. */
typedef struct pkv_pool {
    void *k;
    void *v;
    int64_t num_blocks;
    int64_t num_layers;
    int64_t block_size;
    int64_t num_kv_heads;
    int64_t head_dim;
    int32_t dtype;
    int32_t reserved;
    int64_t block_stride;
    void *k_scale;
    void *v_scale;
} pkv_pool;

/*
 * kv_slot_mapping -- the slot of every new token [P2 sec. 2.2: slot =
 * block_table[block index] * block_size + position inside the block, int64,
 * -1 = padding], with the first-block offset of [P3 sec. 2.2].
 *
 *   block_tables  device int32 [num_seqs, bt_stride]
 *   offsets       device int32 [num_seqs]
 *   token_seq     device int32 [num_tokens]: sequence of token i, or -1 for
 *                 a padding row
 *   token_pos     device int32 [num_tokens]: logical position of token i in
 *                 its sequence
 *   slot_mapping  device int64 [num_tokens], written:
 *                 table[seq][(off+pos)/bs]*bs + (off+pos)%bs, or -1 for a
 *                 padding row or a position outside the table
 * Errors: PKV_ERR_NULL, PKV_ERR_SHAPE (sizes < 0, block_size not a power of
 * two), PKV_ERR_LAUNCH.  num_tokens == 0 enqueues nothing.
 */
PKV_API int kv_slot_mapping(const int32_t *block_tables, int32_t bt_stride,
                            const int32_t *offsets, int32_t num_seqs,
                            const int32_t *token_seq, const int32_t *token_pos,
                            int64_t num_tokens, int32_t block_size,
                            int64_t *slot_mapping, void *stream);

/*
 * kv_scatter -- write new K/V rows into the pool at `layer`
 * [P1 "relation to step14_1": kv_pool[blocks, slots] = K; P2 sec. 2.2:
 * writes indexed (block_id, layer, offset inside block), slot -1 = padding].
 *
 *   k_src, v_src  device [num_tokens, num_kv_heads, head_dim], pool dtype
 *                 (bfloat16 for a quantised pool, each (token, kv head)
 *                 row quantised on write), contiguous.  v_src may be NULL
 *                 to write K only (then the pool's v may be NULL too).
 *   slot_mapping  device int64 [num_tokens]; row i goes to block slot/bs,
 *                 slot slot%bs.  Negative or out-of-pool slots are skipped.
 * Only the addressed rows of `layer` are written; every other byte of the
 * pool is left as it was.  Duplicate slots are a caller error (the row that
 * lands last is unspecified).
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _LAUNCH.
 */
PKV_API int kv_scatter(const pkv_pool *pool, int32_t layer,
                       const void *k_src, const void *v_src,
                       const int64_t *slot_mapping, int64_t num_tokens,
                       void *stream);

/*
 * kv_append -- kv_slot_mapping and kv_scatter in one pass: row i of
 * k_src/v_src is written at the slot of logical position token_pos[i] of
 * sequence token_seq[i] [P2 sec. 2.2 slot_mapping; P3 sec. 2.2 offset;
 * P1 "relation to step14_1"], with exactly the slot kv_slot_mapping
 * computes and the skipping rules of both (token_seq < 0, a position
 * outside the table, a slot outside the pool).  The decode step's write of
 * the new tokens, as one kernel instead of two.
 *
 *   k_src, v_src  as for kv_scatter (v_src may be NULL)
 *   block_tables, bt_stride, offsets, num_seqs, token_seq, token_pos,
 *   num_tokens    as for kv_slot_mapping (block_size is the pool's)
 *   slot_mapping_out  device int64 [num_tokens] receiving the slots (-1 for
 *                 skipped rows), or NULL
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _LAUNCH.
 * num_tokens == 0 enqueues nothing.
 */
PKV_API int kv_append(const pkv_pool *pool, int32_t layer,
                      const void *k_src, const void *v_src,
                      const int32_t *block_tables, int32_t bt_stride,
                      const int32_t *offsets, int32_t num_seqs,
                      const int32_t *token_seq, const int32_t *token_pos,
                      int64_t num_tokens, int64_t *slot_mapping_out,
                      void *stream);

/*
 * kv_gather -- contiguous K/V of each sequence from its block table
 * [P1 "Problem" and "Solution": pool[table[pos/bs], pos%bs] -> (seq_len,
 * num_heads, head_dim); P3 sec. 2.2: reads start at the first-block offset].
 *
 *   block_tables   device int32 [num_seqs, bt_stride]
 *   seq_lens       device int32 [num_seqs]
 *   offsets        device int32 [num_seqs], each in [0, block_size)
 *   out_row_start  device int64 [num_seqs]: first output row of each
 *                  sequence (rows of different sequences must not overlap)
 *   max_seq_len    host bound on every seq_len (sizes the grid)
 *   k_out, v_out   device [out_rows, num_kv_heads, head_dim]; row
 *                  out_row_start[s] + t receives logical token t of s.
 *                  v_out may be NULL to gather K only.
 *   out_rows       rows k_out (and v_out) can hold; a row that would land
 *                  outside [0, out_rows) is not written.
 * A token whose table entry is missing or out of range reads as a zero row.
 * A quantised pool gathers bfloat16 rows bf16(code * scale).
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _LAUNCH.
 */
PKV_API int kv_gather(const pkv_pool *pool, int32_t layer,
                      const int32_t *block_tables, int32_t bt_stride,
                      const int32_t *seq_lens, const int32_t *offsets,
                      const int64_t *out_row_start, int32_t num_seqs,
                      int32_t max_seq_len, void *k_out, void *v_out,
                      int64_t out_rows, void *stream);

/* split_tokens value that asks paged_attn_decode for the device-planned
 * split schedule, and the value paged_attn_decode_schedule returns for it */
#define PKV_SPLIT_PLANNED (-2)
#define PKV_SCHEDULE_PLANNED 1

/*
 * paged_attn_decode_split_tokens -- the split size (tokens per work item)
 * of the split schedule for a bf16 pool when paged_attn_decode is called
 * with split_tokens = 0 and does not take the planned schedule (see
 * paged_attn_decode_schedule, which also gives the choice for fp32 and
 * int8 pools: with fewer (sequence, kv head) pairs than twice the
 * compute units, those stop growing the split at 1024 positions once
 * there are 2 workgroups per compute unit).  A power of two of at least
 * 64 positions: grown while the work items (sequence, kv head, split of
 * max_seq_len tokens) exceed 8 per compute unit (32 with at least two
 * pairs per compute unit), up to 256 positions while at least 2 items per
 * compute unit remain, and for few pairs past 1024 positions while they
 * exceed 4 per compute unit; never past the first split that covers
 * max_seq_len.  Depends on the sizes and on the current device's
 * compute-unit count (256 is assumed when no device can be queried).
 * Returns a positive multiple of 16, or a negative status for bad sizes.
 */
PKV_API int32_t paged_attn_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                               int32_t max_seq_len, int32_t block_size);

/*
 * paged_attn_decode_schedule -- which work schedule paged_attn_decode takes
 * for these sizes, pool dtype (PKV_F32 / PKV_BF16 / PKV_I8 / PKV_I4) and
 * split_tokens:
 *   > 0  the split schedule with this many tokens per split: one workgroup
 *        per (sequence, split of split_tokens flat positions, group of kv
 *        heads);
 *     1  (PKV_SCHEDULE_PLANNED) the device-planned split schedule: the
 *        split schedule with a split size the kernel picks from the actual
 *        lengths, the smallest multiple of 16 (at least 64 positions, and
 *        enough for 16 splits per sequence of max_seq_len) whose
 *        (sequence, split, kv-head group) pieces fit 2 workgroups per
 *        compute unit; pieces of exactly that many positions take the
 *        first workgroups, shorter first and last pieces the last ones.
 *        Taken for bf16 and int8 pools when split_tokens = 0 or PKV_SPLIT_PLANNED
 *        and the batch allows it: at most 64 sequences, at most
 *        compute units / 2 (sequence, kv-head group) pairs, and
 *        max_seq_len / 2 + 32 <= the largest split (split_tokens limit
 *        below);
 *   < 0  a status for bad sizes or dtype (PKV_ERR_UNSUPPORTED for a
 *        planned request the batch or the pool dtype does not allow).
 * All compute the same function; they differ only in fp32 rounding order.
 */
PKV_API int32_t paged_attn_decode_schedule(int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_seq_len, int32_t block_size,
                                           int32_t dtype, int32_t split_tokens);

/*
 * paged_attn_decode_workspace_size -- bytes of device workspace that
 * paged_attn_decode needs for these sizes and this split_tokens.  With
 * split_tokens = 0 it covers the schedule taken for any pool dtype.  0 means no workspace is
 * needed (every sequence fits one split).  Returns (size_t)-1 for bad
 * sizes.
 */
PKV_API size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                                int32_t num_q_heads, int32_t head_dim,
                                                int32_t max_seq_len, int32_t block_size,
                                                int32_t split_tokens);

/*
 * paged_attn_decode -- one decode step of attention for every sequence,
 * reading K/V in place through the block tables (the fused paged kernel of
 * [P1 "comparison with vLLM"; P3 sec. 3.1]: the result of gather followed
 * by standard attention [P2 sec. 2.3], without the gathered copy).
 *
 * For sequence s and query head h, with G = num_q_heads/num_kv_heads and kv
 * head g = h / G (contiguous query-head groups):
 *   out[s,h,:] = softmax_t(scale * q[s,h,:] . K_t[g,:]) . V_t[g,:]
 * over the seq_lens[s] logical tokens t (no causal mask: the one query sees
 * every cached token).  Accumulation is fp32; out is rounded (nearest-even)
 * to the pool dtype.  A sequence of length 0 gives zeros.
 *
 *   q             device [num_seqs, num_q_heads, head_dim], pool dtype
 *   block_tables, seq_lens, offsets  as for kv_gather
 *   max_seq_len   host bound on every seq_len
 *   scale         softmax scale (e.g. 1/sqrt(head_dim))
 *   split_tokens  0 = automatic (see paged_attn_decode_schedule);
 *                 PKV_SPLIT_PLANNED = the device-planned split schedule
 *                 (limits as above, else PKV_ERR_UNSUPPORTED); else the
 *                 tokens per split-K work item, a positive multiple of 16
 *                 with split_tokens/block_size + 2 <= 1024.  A sequence
 *                 spread over several work items is computed as partial
 *                 softmaxes, merged (log-sum-exp) by the work item that
 *                 finishes last (or, past 16 splits, by a second kernel),
 *                 in a fixed order; the partition depends only on the
 *                 sizes, the lengths and offsets, and the device's
 *                 compute-unit count, so results are bitwise reproducible
 *                 run to run.  A sequence longer than max_seq_len is
 *                 attended over its first max_seq_len tokens and an offset
 *                 outside [0, block_size) is clamped into it, in every
 *                 schedule (both break the contract; no access leaves the
 *                 buffers, and the workspace stays reusable).
 *   out           device [num_seqs, num_q_heads, head_dim], pool dtype
 *   workspace     device scratch of at least
 *                 paged_attn_decode_workspace_size(...) bytes (may be NULL
 *                 when that size is 0).  It must be all zero before its
 *                 first use (e.g. one hipMemset after allocation); each call
 *                 leaves its counters zero again, so a workspace is reused
 *                 as is.  Calls that share a workspace must not overlap
 *                 (issue them on one stream).
 * Supported: head_dim in {64, 128}, G in {1, 2, 4, 8}.  A quantised pool
 * takes bfloat16 q and out, runs the split or the planned schedule and
 * attends to the stored values code * scale.
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _WORKSPACE,
 * _UNSUPPORTED, _LAUNCH.
 */
PKV_API int paged_attn_decode(const pkv_pool *pool, int32_t layer,
                              const void *q, int32_t num_q_heads,
                              const int32_t *block_tables, int32_t bt_stride,
                              const int32_t *seq_lens, const int32_t *offsets,
                              int32_t num_seqs, int32_t max_seq_len, float scale,
                              int32_t split_tokens, void *out,
                              void *workspace, size_t workspace_bytes,
                              void *stream);

/* Bytes of the fixed per-device scratch of paged_attn_decode_noalloc. */
#define PKV_NOALLOC_SCRATCH_BYTES (32u << 20)

/*
 * paged_attn_decode_noalloc -- paged_attn_decode without a workspace
 * argument, for callers that cannot allocate device memory around a call:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  It allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine).
 *
 * The split partials and merge counters live in a fixed array of
 * PKV_NOALLOC_SCRATCH_BYTES (32 MiB) of device memory inside the library;
 * every device the library runs on holds its own copy until the process
 * ends (its address is looked up once per device, on that device's first
 * call).  Each call first clears the merge counters it uses (a small fill
 * kernel on `stream`, not a memset), then runs exactly the kernels and
 * schedule paged_attn_decode runs for the same arguments: the output is
 * bitwise the output of paged_attn_decode with a workspace.
 *
 * Every call on a device shares that device's array, which keeps the last
 * call's contents: calls that overlap on one device (issued on different
 * streams, or from several threads without ordering) race on it and may
 * return wrong results.  Issue them on one stream.
 *
 * Arguments: as paged_attn_decode, without workspace / workspace_bytes.
 * Errors: as paged_attn_decode; PKV_ERR_SCRATCH (nothing enqueued) when
 * paged_attn_decode_workspace_size(...) for these sizes and split_tokens
 * exceeds PKV_NOALLOC_SCRATCH_BYTES; PKV_ERR_DEVICE when the array's device
 * address cannot be looked up on the current device.
 */
PKV_API int paged_attn_decode_noalloc(const pkv_pool *pool, int32_t layer,
                                      const void *q, int32_t num_q_heads,
                                      const int32_t *block_tables, int32_t bt_stride,
                                      const int32_t *seq_lens, const int32_t *offsets,
                                      int32_t num_seqs, int32_t max_seq_len, float scale,
                                      int32_t split_tokens, void *out, void *stream);

/*
 * paged_attn_decode_append -- one whole decode step in one call (one launch
 * on a float pool): each sequence's new token is written into the pool, then
 * attended to with the rest.  For every sequence s with seq_lens[s] > 0, the new token sits at
 * logical position seq_lens[s] - 1 (its K/V row is already counted in
 * seq_lens): its slot is block_tables[s][(p)/block_size] * block_size +
 * p % block_size with p = offsets[s] + seq_lens[s] - 1 [P2 sec. 2.2 slot
 * formula; P3 sec. 2.2 offset], and
 *   K pool [slot/bs, layer, slot%bs, :, :] = k_new[s, :, :]
 *   V pool [slot/bs, layer, slot%bs, :, :] = v_new[s, :, :]
 * exactly as kv_append with token_seq[s] = s, token_pos[s] = seq_lens[s]-1
 * writes them [P1 "relation to step14_1" scatter]; out is then what
 * paged_attn_decode computes over tokens 0 .. seq_lens[s]-1 of the updated
 * pool.  A table entry of -1 at that position writes nothing (the
 * position is masked, as in decode), and neither does a sequence whose
 * length or offset breaks the contract (seq_lens[s] > max_seq_len, offset
 * outside [0, block_size)): it is attended as paged_attn_decode clamps it.  The write happens inside the
 * attention kernel, by the work item whose range ends the sequence, before
 * it reads that row; no other work item reads it.
 * On a quantised pool the new rows are quantised as kv_append quantises
 * them (one scale per row and kv head, round-half-even codes) and written
 * by a first launch, which skips the same sequences; decode then runs as a
 * second launch on the same stream.
 *
 *   k_new, v_new  device [num_seqs, num_kv_heads, head_dim], 16-byte aligned,
 *                 both required: the pool dtype (float pools) or bf16
 *                 (quantised pools)
 *   everything else as for paged_attn_decode (same workspace size)
 * Errors: as paged_attn_decode; PKV_ERR_NULL when k_new or v_new is NULL.
 */
PKV_API int paged_attn_decode_append(const pkv_pool *pool, int32_t layer,
                                     const void *q, int32_t num_q_heads,
                                     const void *k_new, const void *v_new,
                                     const int32_t *block_tables, int32_t bt_stride,
                                     const int32_t *seq_lens, const int32_t *offsets,
                                     int32_t num_seqs, int32_t max_seq_len, float scale,
                                     int32_t split_tokens, void *out,
                                     void *workspace, size_t workspace_bytes,
                                     void *stream);

/*
 * paged_attn_prefill -- prefill / append attention: the queries of
 * sequence s are its last n_s = q_start[s+1] - q_start[s] cached tokens
 * (their K/V already written, e.g. by kv_append) [P2 sec. 2.4 "prefill
 * batch"]; query i of s sits at logical position P = seq_lens[s] - n_s + i
 * and attends causally to the sequence's tokens 0 .. P, read in place
 * through its block table and first-block offset [P3 sec. 2.2] -- so a
 * request whose first blocks are a shared prefix attends to them without a
 * copy.  For query head h (kv head h / G, as for decode):
 *   out[row,h,:] = softmax_t<=P(scale * q[row,h,:] . K_t) . V_t
 * fp32 accumulation, out rounded to the pool dtype.  A query with P < 0
 * (more queries than tokens) gives zeros.  n_s = 1 is paged_attn_decode.
 *
 *   q, out        device [num_q_rows, num_q_heads, head_dim], pool dtype
 *   q_start       device int32 [num_seqs + 1]: q_start[0] = 0, nondecreasing,
 *                 q_start[num_seqs] = num_q_rows (caller contract)
 *   max_q_len     host bound on every n_s (rows of a sequence past it are
 *                 left unwritten)
 *   block_tables, seq_lens, offsets  as for paged_attn_decode
 * Supported: head_dim in {64, 128}, G in {1, 2, 4, 8}; float pools only
 * (PKV_ERR_UNSUPPORTED for a quantised pool).
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _UNSUPPORTED, _LAUNCH.
 */
PKV_API int paged_attn_prefill(const pkv_pool *pool, int32_t layer,
                               const void *q, int32_t num_q_heads,
                               const int32_t *q_start, int32_t num_q_rows, int32_t max_q_len,
                               const int32_t *block_tables, int32_t bt_stride,
                               const int32_t *seq_lens, const int32_t *offsets,
                               int32_t num_seqs, float scale, void *out, void *stream);

/*
 * kv_read_blocks -- a read-rate reference, not part of the pages' method:
 * for i < num_ids, reads the layer-`layer` slice (block_size rows of all kv
 * heads, contiguous) of K and of V of block block_ids[i] and writes the
 * XOR of all their 32-bit words to out[i].  The slices are the bytes paged
 * decode attention reads for those blocks, so timing this call gives the
 * read rate the decode kernels are compared with.
 *   block_ids     device int32 [num_ids]; an id outside [0, num_blocks)
 *                 reads nothing and gives 0
 *   out           device uint32 [num_ids]
 * V is read when pool->v is set.  For a quantised pool the codes are read
 * (not the scales).  Asynchronous on `stream`.
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _LAYER, _ALIGN, _LAUNCH.
 */
PKV_API int kv_read_blocks(const pkv_pool *pool, int32_t layer, const int32_t *block_ids,
                           int64_t num_ids, uint32_t *out, void *stream);

/*
 * kv_copy_blocks -- whole-block copies: for i < num_pairs, every layer of K
 * and of V of block src_blocks[i] is copied to block dst_blocks[i] (codes
 * and scales for a quantised pool).  This
 * is the copy of copy-on-write [P3 sec. 3.1: vLLM shares blocks by
 * copy-on-write + ref_count; sec. 2.4 ref_count]: before a sequence writes
 * into a block other tables also hold, it takes a new block (pkv_bm_cow)
 * and the block's contents are copied here.
 *
 *   src_blocks, dst_blocks  device int32 [num_pairs]; a pair with an id
 *                 outside [0, num_blocks) is skipped.  Destinations must be
 *                 distinct and none may be another pair's source (caller
 *                 contract; pkv_bm_cow's pairs meet it).
 * V is copied when pool->v is set.  Asynchronous on `stream`.
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _ALIGN, _LAUNCH.
 */
PKV_API int kv_copy_blocks(const pkv_pool *pool, const int32_t *src_blocks,
                           const int32_t *dst_blocks, int64_t num_pairs, void *stream);

/*
 * kv_swap_out / kv_swap_in -- move whole blocks between the pool and host
 * memory: the swap of preemption [P2 sec. 2.4: when free blocks run short
 * the scheduler can move a sequence's KV from GPU to CPU, or drop it and
 * recompute].  Block i of the list is one dense block per tensor
 * (num_layers * block_size * num_kv_heads * head_dim elements) at
 * k_host / v_host + i * that many bytes.
 *
 *   block_ids     HOST int32 [n], each in [0, num_blocks), else
 *                 PKV_ERR_BLOCK before any copy
 *   k_host, v_host  host buffers of n dense blocks each; v_host is used
 *                 (and required) when pool->v is set.  For a quantised
 *                 pool each buffer holds the n blocks' codes, then the n
 *                 blocks' scales (num_layers * num_kv_heads * block_size
 *                 floats per block).  Pinned host memory
 *                 (hipHostMalloc, torch pin_memory) keeps the copies
 *                 asynchronous on `stream`; pageable memory works, but the
 *                 copies then finish before the call returns.
 * Runs of consecutive ids in a dense pool move as one copy.
 * Errors: PKV_ERR_NULL, _DTYPE, _SHAPE, _ALIGN, _BLOCK, _LAUNCH.
 */
PKV_API int kv_swap_out(const pkv_pool *pool, const int32_t *block_ids, int64_t n,
                        void *k_host, void *v_host, void *stream);
PKV_API int kv_swap_in(const pkv_pool *pool, const int32_t *block_ids, int64_t n,
                       const void *k_host, const void *v_host, void *stream);

/*
 * kv_validate -- count violations of the caller contract, for debugging:
 * offsets outside [0, block_size); seq_len < 0, > max_seq_len (when
 * max_seq_len >= 0) or > the table's capacity bt_stride*block_size - offset
 * [P3 sec. 2.2]; block ids outside [0, num_blocks) among the entries a
 * sequence uses; slots that are neither -1 nor inside the pool
 * [P2 sec. 2.2].  Tables or slot_mapping may be NULL (with num_seqs or
 * num_tokens 0) to skip that part.
 *   violations  device int64 [1]: zeroed, then incremented by the kernels
 *               (asynchronous; read it after the stream completes).
 * Errors: PKV_ERR_NULL, _SHAPE, _LAUNCH.
 */
PKV_API int kv_validate(const pkv_pool *pool, const int32_t *block_tables,
                        int32_t bt_stride, const int32_t *seq_lens,
                        const int32_t *offsets, int32_t num_seqs,
                        int32_t max_seq_len, const int64_t *slot_mapping,
                        int64_t num_tokens, int64_t *violations, void *stream);

/* pkv_status_string -- static text for a status code (never NULL). */
PKV_API const char *pkv_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
