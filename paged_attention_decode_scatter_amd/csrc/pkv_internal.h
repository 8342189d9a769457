// pkv_internal.h -- argument blocks and launchers shared by the HIP sources
// of libpagedkv.so (not part of the public ABI; see include/pagedkv.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

// Tokens one wavefront of the decode kernel consumes per iteration.
constexpr int kChunkTokens = 16;
// Block-table entries a decode or gather workgroup stages in LDS.
constexpr int kBtLds = 1024;
// Most splits per sequence (the merge pass keeps one weight per split in
// LDS).
constexpr int kMaxSplits = 4096;
// Gather/scatter workgroup size.
constexpr int kCopyThreads = 256;

// A pool as the kernels see it: byte addresses of (block b, layer, slot s)
// rows are base + b*block_stride + layer_off + s*row_bytes.
struct PoolView {
    const char *k;
    const char *v;
    int64_t block_stride;  // num_layers * block_size * row_bytes
    int64_t layer_off;     // layer * block_size * row_bytes
    int32_t row_bytes;     // num_kv_heads * head_dim * element size
    int32_t num_blocks;
    int32_t lbs;           // log2(block_size)
    int32_t pad_;
    // quantised pools: the scales of this layer; the scale of (block b,
    // kv head h, slot r) is ks[b * sc_block + h * block_size + r]
    const float *ks;
    const float *vs;
    int64_t sc_block;      // num_layers * num_kv_heads * block_size
};

struct SlotArgs {
    const int32_t *block_tables;
    const int32_t *offsets;
    const int32_t *token_seq;
    const int32_t *token_pos;
    int64_t *slots;
    int64_t num_tokens;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t lbs;
};

struct ScatterArgs {
    char *kpool;
    char *vpool;
    const char *k_src;
    const char *v_src;
    const int64_t *slots;
    int64_t num_tokens;
    int64_t total_slots;   // num_blocks * block_size
    int64_t block_stride;
    int64_t layer_off;
    int32_t row_bytes;
    int32_t lbs;
    int32_t tok_per_wg;
    int32_t lcpr;          // log2(row_bytes/16), or -1 if not a power of two
};

// Slot computation and scatter in one pass (kv_append).
struct AppendArgs {
    ScatterArgs sc;              // slots unused; everything else as for the scatter
    const int32_t *block_tables;
    const int32_t *offsets;
    const int32_t *token_seq;
    const int32_t *token_pos;
    int64_t *slots_out;          // may be null
    int32_t bt_stride;
    int32_t num_seqs;
};

// Quantising scatter (int8 pools): bfloat16 rows in, codes and scales out.
// slots == null: the slots are computed as kv_append computes them.
struct ScatterQ8Args {
    char *kpool;
    char *vpool;
    float *ks;             // scales of the layer, as PoolView::ks
    float *vs;
    const char *k_src;
    const char *v_src;
    const int64_t *slots;
    const int32_t *block_tables;
    const int32_t *offsets;
    const int32_t *token_seq;
    const int32_t *token_pos;
    int64_t *slots_out;    // may be null
    // decode-step mode (slots and token_seq null): token s is sequence s's
    // new token, at position step_lens[s] - 1; nothing is written for a
    // length outside [1, step_max_len] or an offset outside [0, block_size)
    const int32_t *step_lens;
    int32_t step_max_len;
    int64_t num_tokens;
    int64_t total_slots;
    int64_t block_stride;
    int64_t layer_off;
    int64_t sc_block;
    int32_t num_kv_heads;
    int32_t head_dim;
    int32_t lbs;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t qbits;         // bits per code: 8 (int8 pool) or 4 (int4 pool)
};

struct GatherArgs {
    PoolView pool;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    const int32_t *offsets;
    const int64_t *out_row_start;
    char *k_out;
    char *v_out;
    int64_t out_rows;      // rows k_out/v_out can hold; rows beyond are skipped
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t tok_per_wg;
    int32_t tiles_per_seq;
    int32_t lcpr;
};

struct DecodeArgs {
    PoolView pool;
    const char *q;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    const int32_t *offsets;
    char *out;
    const char *k_new;     // decode with append: [num_seqs][num_kv_heads][head_dim] new rows
    const char *v_new;     //   (position seq_len - 1); null for plain decode
    uint32_t *ws_cnt;      // [num_seqs][head_groups] finished splits (zero between calls)
    float *ws_ml;          // [num_seqs][max_splits][num_q_heads][2]  (m, l)
    float *ws_acc;         // [num_seqs][max_splits][num_q_heads][head_dim] floats; the in-kernel merge's
                           // records of the MFMA kernels at head_dim 128 use the same indexing in halves
    float scale_log2;      // scale * log2(e): scores live in the exp2 domain
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t split_tokens;
    int32_t max_splits;
    int32_t heads_per_wg;
    int32_t head_groups;
    int32_t fused_merge;   // 1: the last split of a (sequence, head group) merges; 0: merge kernel
    int32_t plan;          // > 0: device-planned split, this many workgroups (split_tokens: the smallest split)
    int32_t max_len;       // the caller's max_seq_len (device-planned split clamps to it)
};

// Most splits per sequence merged by the last finishing workgroup; beyond
// this a separate, wider merge kernel is faster.
constexpr int kFusedMergeMaxSplits = 16;

// Device-planned split schedule: at most this many sequences (one per lane
// of the wavefront that plans).
constexpr int kPlanMaxSeqs = 64;

// Prefill / append attention: the last n_s = q_start[s+1] - q_start[s]
// tokens of sequence s are its queries (rows q_start[s].. of q and out).
// Prefill (bf16 kernel) workgroups: kPrefillWaves<G> = max(4, G)
// wavefronts, G query heads x kPrefillWaves<G> / G query groups, sharing
// every staged key chunk.  A wavefront holds kPrefillWaveQueries queries
// (sub-tiles of 16), as many as fit two wavefronts per SIMD without spills;
// a workgroup tile is kPrefillTile queries.  Measured on MI355X
// (prefix-sharing batch, every suffix token a query, head_dim 128, G 4): 16
// queries per wavefront 11.2 ms, 32: 8.3 ms, 48: 7.1 ms (64 spills); the
// depth of the key ring (3 to 8 chunks) changed nothing; 4 wavefronts per
// workgroup (two workgroups per CU, whose barriers do not line up) 6.59 ms
// against 6.88 ms with 8 (one per CU), same process.
template <int G>
inline constexpr int kPrefillWaves = G > 4 ? G : 4;
inline int prefill_waves(int64_t group) { return group > 4 ? (int)group : 4; }
#ifndef PKV_PREFILL_WQ64
#define PKV_PREFILL_WQ64 64
#endif
#ifndef PKV_PREFILL_WQ128
#define PKV_PREFILL_WQ128 48
#endif
#ifndef PKV_PREFILL_VSWZ
#define PKV_PREFILL_VSWZ 1
#endif
#ifndef PKV_PREFILL_RING
#define PKV_PREFILL_RING 6
#endif
// key chunks staged in LDS: three stages of two 16-key chunks, one barrier
// per stage, loads issued two stages ahead (two chunks per barrier: 6.30 ms
// against 6.61 ms with one chunk per barrier and a ring of 3, same process)
constexpr int kPrefillRing = PKV_PREFILL_RING;
template <int D, int G>
inline constexpr int kPrefillWaveQueries = D == 64 ? PKV_PREFILL_WQ64 : PKV_PREFILL_WQ128;
template <int D, int G>
inline constexpr int kPrefillTile = kPrefillWaveQueries<D, G> * (kPrefillWaves<G> / G);
inline int prefill_tile(int64_t head_dim, int64_t group) {
    return (head_dim == 64 ? PKV_PREFILL_WQ64 : PKV_PREFILL_WQ128) * (prefill_waves(group) / (int)group);
}

struct PrefillArgs {
    PoolView pool;
    const char *q;
    const int32_t *q_start;
    const int32_t *block_tables;
    const int32_t *seq_lens;
    const int32_t *offsets;
    char *out;
    float scale_log2;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_kv_heads;
    int32_t num_q_heads;
    int32_t num_q_rows;
    int32_t q_tiles;       // query tiles (prefill_tile queries) per sequence in the grid
    int32_t max_q_len;     // queries past it in a sequence are not computed
    int32_t heads_per_wg;  // fp32 kernel: kv heads per workgroup
    int32_t head_groups;
    int32_t seg_chunks;    // most 16-position chunks staged at once
};

// Whole-block copies (copy-on-write): one workgroup per (pair, piece of
// kCopyBlockPiece bytes of the block).
constexpr int64_t kCopyBlockPiece = 64 * 1024;
struct CopyBlocksArgs {
    char *k;
    char *v;
    const int32_t *src;
    const int32_t *dst;
    int64_t num_pairs;
    int64_t num_blocks;
    int64_t block_bytes;   // one block of one tensor, all layers
    int64_t block_stride;
    int64_t pieces;        // ceil(block_bytes / kCopyBlockPiece)
};

// Read-rate reference: the layer slices of listed blocks, read and folded
// into one checksum per block.
struct ReadBlocksArgs {
    const char *k;
    const char *v;         // may be null
    const int32_t *ids;
    uint32_t *out;
    int64_t n;
    int64_t num_blocks;
    int64_t block_stride;
    int64_t layer_off;
    int64_t slice_bytes;   // block_size * row_bytes
};

struct ValidateArgs {
    const int32_t *block_tables;
    const int32_t *seq_lens;
    const int32_t *offsets;
    const int64_t *slots;
    unsigned long long *count;
    int64_t num_tokens;
    int64_t total_slots;
    int32_t bt_stride;
    int32_t num_seqs;
    int32_t num_blocks;
    int32_t block_size;
    int32_t max_seq_len;
};

hipError_t launch_slot_mapping(const SlotArgs &a, hipStream_t s);
hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, hipStream_t s);
bool prefill_supported(int dtype, int head_dim, int group);
hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, int group, hipStream_t s);
hipError_t launch_gather(const GatherArgs &a, hipStream_t s);
hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t s);
hipError_t launch_scatter_q8(const ScatterQ8Args &a, hipStream_t s);
hipError_t launch_gather_q8(const GatherArgs &a, int head_dim, int qbits, hipStream_t s);
hipError_t launch_validate(const ValidateArgs &a, hipStream_t s);
hipError_t launch_read_blocks(const ReadBlocksArgs &a, hipStream_t s);
hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s);
// Returns hipErrorInvalidValue when (dtype, head_dim, group) is not built.
hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, int group,
                         hipStream_t s);
bool decode_supported(int dtype, int head_dim, int group);

}  // namespace pkv
