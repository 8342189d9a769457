/*
 * pagedkv_oracle.c -- plain, slow, obviously-correct CPU oracle for
 * block-table-indirected access to a paged KV cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: it exists so that tests, the smoke check and the CPU
 * baseline leg of the benchmark have an independent answer to compare the
 * HIP kernels against.  It shares no code, header, table or constant with
 * the HIP library (the only thing both sides see are the seeded inputs).
 *
 * Sources (three web pages on paged KV caches):
 *   [P1] mini-vllm tutorial, "step14_2 - index_select gather"
 *   [P2] "vLLM PagedAttention source notes" (minivLLM Task 6 background)
 *   [P3] mini-runtime, chapter 12 "Paged KV Cache"
 *
 * Pool layout (both K and V, separate arrays) [P2 sec. 2.2]:
 *   (num_blocks, num_layers, block_size, num_kv_heads, head_dim)
 * One "row" is the num_kv_heads*head_dim elements of one token at one layer;
 * the oracle moves rows as bytes, so scatter and gather are dtype-agnostic.
 *
 * Element types: 0 = float32, 1 = bfloat16 (the upper 16 bits of an
 * IEEE float32).  Floating-point arithmetic is done in double.
 *
 * Every function returns a negative value when its inputs break the
 * caller contract (the oracle refuses rather than guesses).
 *
 * Parity pins (what ties each function to the pages rather than to itself)
 * live in the CPU tests; each function below names the passage it follows.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1

static int64_t elem_size(int dtype) { return dtype == ORC_BF16 ? 2 : 4; }

/* Decode one stored element to double.  bf16 -> float is exact (the value
 * is the float whose upper half is the stored 16 bits). */
static double load_elem(const uint8_t *p, int dtype) {
    if (dtype == ORC_BF16) {
        uint16_t h;
        memcpy(&h, p, 2);
        uint32_t bits = ((uint32_t)h) << 16;
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    float f;
    memcpy(&f, p, 4);
    return (double)f;
}

/* Address of (block b, layer, slot s) row inside a pool. */
static int64_t row_index(int64_t b, int64_t num_layers, int64_t layer,
                         int64_t block_size, int64_t s) {
    return (b * num_layers + layer) * block_size + s;
}

/* ------------------------------------------------------------------------
 * Slot computation.
 * [P2 sec. 2.2]: slot_mapping is int64, one entry per token, -1 = padding;
 *   slot = block_table[block_idx] * block_size + (position inside block).
 * [P3 sec. 2.2]: a BlockTable carries a first-block start offset; logical
 *   token t therefore sits at flat position offset + t of its table.
 * Token i belongs to sequence token_seq[i] (-1 = padding row) at logical
 * position token_pos[i].
 * Returns 0, or -1 if a token's position falls outside its table.
 * ---------------------------------------------------------------------- */
int64_t orc_slot_mapping(const int32_t *block_tables, int64_t bt_stride,
                         const int32_t *offsets, int64_t num_seqs,
                         const int32_t *token_seq, const int32_t *token_pos,
                         int64_t num_tokens, int64_t block_size,
                         int64_t *slot_mapping) {
    for (int64_t i = 0; i < num_tokens; i++) {
        int64_t seq = token_seq[i];
        if (seq < 0) {
            slot_mapping[i] = -1;
            continue;
        }
        if (seq >= num_seqs || token_pos[i] < 0) return -1;
        int64_t p = (int64_t)offsets[seq] + (int64_t)token_pos[i];
        int64_t block_idx = p / block_size;
        int64_t in_block = p % block_size;
        if (block_idx >= bt_stride) return -1;
        int64_t phys = block_tables[seq * bt_stride + block_idx];
        if (phys < 0) return -1;
        slot_mapping[i] = phys * block_size + in_block;
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Scatter ("write", the mirror of the gather) [P1 "relation to step14_1"]:
 * kv_pool[physical_block, slot] = K.  Written into (block, layer, slot)
 * [P2 sec. 2.2]; slot -1 is padding and is skipped [P2 sec. 2.2].
 * Tokens are applied in order, so with duplicate slots the last one wins.
 * Returns 0, or -1 on a slot that is neither -1 nor inside the pool.
 * ---------------------------------------------------------------------- */
int64_t orc_scatter(uint8_t *pool, int64_t num_blocks, int64_t num_layers,
                    int64_t block_size, int64_t row_bytes, int64_t layer,
                    const uint8_t *src, const int64_t *slot_mapping,
                    int64_t num_tokens) {
    if (layer < 0 || layer >= num_layers) return -1;
    for (int64_t i = 0; i < num_tokens; i++) {
        int64_t slot = slot_mapping[i];
        if (slot == -1) continue;
        if (slot < 0 || slot >= num_blocks * block_size) return -1;
        int64_t b = slot / block_size;
        int64_t s = slot % block_size;
        memcpy(pool + row_index(b, num_layers, layer, block_size, s) * row_bytes,
               src + i * row_bytes, (size_t)row_bytes);
    }
    return 0;
}

/* ------------------------------------------------------------------------
 * Gather, as the loop-and-cat definition [P1 "Problem"]: walk the table's
 * block ids in logical order, take min(block_size, remaining) rows from
 * each, concatenate.  Extended with the first-block start offset of
 * [P3 sec. 2.2]: the first block contributes rows offset .. and reading
 * from the block head instead would misalign every token.
 * Sequences are concatenated one after another into `out`.
 * Returns the number of rows written, or -1 if a table is too short for
 * its seq_len or names a block outside the pool.
 * ---------------------------------------------------------------------- */
int64_t orc_gather(const uint8_t *pool, int64_t num_blocks, int64_t num_layers,
                   int64_t block_size, int64_t row_bytes, int64_t layer,
                   const int32_t *block_tables, int64_t bt_stride,
                   const int32_t *seq_lens, const int32_t *offsets,
                   int64_t num_seqs, uint8_t *out) {
    if (layer < 0 || layer >= num_layers) return -1;
    int64_t out_rows = 0;
    for (int64_t s = 0; s < num_seqs; s++) {
        int64_t remaining = seq_lens[s];
        int64_t start = offsets[s];
        if (remaining < 0 || start < 0 || start >= block_size) return -1;
        for (int64_t j = 0; remaining > 0; j++) {
            if (j >= bt_stride) return -1;
            int64_t bid = block_tables[s * bt_stride + j];
            if (bid < 0 || bid >= num_blocks) return -1;
            int64_t take = block_size - start;
            if (take > remaining) take = remaining;
            memcpy(out + out_rows * row_bytes,
                   pool + row_index(bid, num_layers, layer, block_size, start) * row_bytes,
                   (size_t)(take * row_bytes));
            out_rows += take;
            remaining -= take;
            start = 0;
        }
    }
    return out_rows;
}

/* ------------------------------------------------------------------------
 * Attention, as "gather, then standard multi-head attention"
 * [P2 sec. 2.3; P3 sec. 3.1: gather into a contiguous tensor, then SDPA].
 * The fused paged kernel only removes the copy [P1 "comparison with vLLM"],
 * so this is the result it must reproduce.
 *
 * Queries of sequence s (L = seq_lens[s] cached tokens):
 *   decode  (q_start == NULL): one query, row s of q, at logical position
 *           L - 1 -- it sees every cached token (no mask);
 *   prefill (q_start given): the rows q_start[s] .. q_start[s+1]-1 of q are
 *           the sequence's last n tokens [P2 sec. 2.4 "prefill batch": the
 *           prompt tokens' K/V are written, then attended]; query i sits at
 *           logical position L - n + i and sees tokens 0 .. L - n + i
 *           (causal).  A query whose position would be negative sees
 *           nothing and yields zeros.
 * For a query at position P and query head h, with G = num_q_heads /
 * num_kv_heads and kv head g = h / G (contiguous GQA groups; G = 1 is MHA):
 *   Kc, Vc = gather(s) restricted to kv head g       (seq_len x head_dim)
 *   score_t = scale * sum_d q[row,h,d] * Kc[t,d]      for t = 0 .. P
 *   w_t     = exp(score_t - max_t score_t)
 *   out[row,h,:] = sum_t w_t * Vc[t,:] / sum_t w_t
 * in double.  A sequence of length 0 yields zeros.
 * q: (rows, num_q_heads, head_dim) in the pool dtype.
 * out: (rows, num_q_heads, head_dim) double.
 * The (s, g) work items are independent; `num_threads` worker threads each
 * take whole items, so threading changes no arithmetic.
 * Returns 0, or -1 on bad arguments.
 * ---------------------------------------------------------------------- */
typedef struct {
    const uint8_t *kpool, *vpool;
    int64_t num_blocks, num_layers, block_size, num_kv_heads, head_dim;
    int dtype;
    int64_t layer;
    const uint8_t *q;
    const int32_t *q_start;   /* NULL: decode */
    int64_t num_q_heads;
    const int32_t *block_tables;
    int64_t bt_stride;
    const int32_t *seq_lens, *offsets;
    int64_t num_seqs;
    double scale;
    double *out;
    int64_t next_item;
    pthread_mutex_t lock;
    int failed;
} decode_job;

/* One work item: sequence s and kv head g.  The sequence is gathered once,
 * then every query of the sequence, for every query head of group g
 * (h = g*G .. g*G+G-1, i.e. h / G == g), attends over its visible tokens. */
static int decode_group(decode_job *J, int64_t s, int64_t g) {
    const int64_t D = J->head_dim;
    const int64_t e = elem_size(J->dtype);
    const int64_t row_bytes = J->num_kv_heads * D * e;
    const int64_t G = J->num_q_heads / J->num_kv_heads;
    const int64_t L = J->seq_lens[s];
    const int64_t n = J->q_start ? (int64_t)J->q_start[s + 1] - J->q_start[s] : 1;
    const int64_t row0 = J->q_start ? J->q_start[s] : s;
    for (int64_t i = 0; i < n; i++)
        for (int64_t h = g * G; h < (g + 1) * G; h++)
            for (int64_t d = 0; d < D; d++) J->out[((row0 + i) * J->num_q_heads + h) * D + d] = 0.0;
    if (L == 0) return 0;

    /* gather the whole sequence (all kv heads) with the definition above */
    uint8_t *krows = (uint8_t *)malloc((size_t)(L * row_bytes));
    uint8_t *vrows = (uint8_t *)malloc((size_t)(L * row_bytes));
    double *score = (double *)malloc((size_t)L * sizeof(double));
    double *num = (double *)malloc((size_t)D * sizeof(double));
    int rc = 0;
    if (!krows || !vrows || !score || !num) { rc = -1; goto done; }
    if (orc_gather(J->kpool, J->num_blocks, J->num_layers, J->block_size, row_bytes,
                   J->layer, J->block_tables + s * J->bt_stride, J->bt_stride,
                   J->seq_lens + s, J->offsets + s, 1, krows) != L ||
        orc_gather(J->vpool, J->num_blocks, J->num_layers, J->block_size, row_bytes,
                   J->layer, J->block_tables + s * J->bt_stride, J->bt_stride,
                   J->seq_lens + s, J->offsets + s, 1, vrows) != L) {
        rc = -1;
        goto done;
    }

    for (int64_t i = 0; i < n; i++) {
        const int64_t P = L - n + i;   /* the query's logical position */
        if (P < 0) continue;           /* sees no token: zeros */
        const int64_t row = row0 + i;
        for (int64_t h = g * G; h < (g + 1) * G; h++) {
            const uint8_t *qh = J->q + (row * J->num_q_heads + h) * D * e;
            double *o = J->out + (row * J->num_q_heads + h) * D;
            double mx = -INFINITY;
            for (int64_t t = 0; t <= P; t++) {
                const uint8_t *kt = krows + t * row_bytes + g * D * e;
                double dot = 0.0;
                for (int64_t d = 0; d < D; d++)
                    dot += load_elem(qh + d * e, J->dtype) * load_elem(kt + d * e, J->dtype);
                score[t] = J->scale * dot;
                if (score[t] > mx) mx = score[t];
            }
            double den = 0.0;
            for (int64_t d = 0; d < D; d++) num[d] = 0.0;
            for (int64_t t = 0; t <= P; t++) {
                double w = exp(score[t] - mx);
                den += w;
                const uint8_t *vt = vrows + t * row_bytes + g * D * e;
                for (int64_t d = 0; d < D; d++) num[d] += w * load_elem(vt + d * e, J->dtype);
            }
            for (int64_t d = 0; d < D; d++) o[d] = num[d] / den;
        }
    }

done:
    free(krows);
    free(vrows);
    free(score);
    free(num);
    return rc;
}

static void *decode_worker(void *arg) {
    decode_job *J = (decode_job *)arg;
    const int64_t total = J->num_seqs * J->num_kv_heads;
    for (;;) {
        pthread_mutex_lock(&J->lock);
        int64_t item = J->next_item++;
        pthread_mutex_unlock(&J->lock);
        if (item >= total) break;
        if (decode_group(J, item / J->num_kv_heads, item % J->num_kv_heads) != 0) {
            pthread_mutex_lock(&J->lock);
            J->failed = 1;
            pthread_mutex_unlock(&J->lock);
        }
    }
    return NULL;
}

static int64_t run_attention(const uint8_t *kpool, const uint8_t *vpool, int64_t num_blocks,
                             int64_t num_layers, int64_t block_size, int64_t num_kv_heads,
                             int64_t head_dim, int64_t dtype, int64_t layer, const uint8_t *q,
                             const int32_t *q_start, int64_t num_q_heads,
                             const int32_t *block_tables, int64_t bt_stride,
                             const int32_t *seq_lens, const int32_t *offsets, int64_t num_seqs,
                             double scale, double *out, int64_t num_threads) {
    if (dtype != ORC_F32 && dtype != ORC_BF16) return -1;
    if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads != 0) return -1;
    if (layer < 0 || layer >= num_layers || head_dim <= 0) return -1;
    decode_job J;
    J.kpool = kpool; J.vpool = vpool;
    J.num_blocks = num_blocks; J.num_layers = num_layers; J.block_size = block_size;
    J.num_kv_heads = num_kv_heads; J.head_dim = head_dim; J.dtype = (int)dtype;
    J.layer = layer; J.q = q; J.q_start = q_start; J.num_q_heads = num_q_heads;
    J.block_tables = block_tables; J.bt_stride = bt_stride;
    J.seq_lens = seq_lens; J.offsets = offsets; J.num_seqs = num_seqs;
    J.scale = scale; J.out = out; J.next_item = 0; J.failed = 0;
    pthread_mutex_init(&J.lock, NULL);
    if (num_threads < 1) num_threads = 1;
    if (num_threads > 256) num_threads = 256;
    pthread_t tid[256];
    int64_t started = 0;
    for (int64_t i = 1; i < num_threads; i++) {
        if (pthread_create(&tid[i], NULL, decode_worker, &J) != 0) break;
        started = i;
    }
    decode_worker(&J);
    for (int64_t i = 1; i <= started; i++) pthread_join(tid[i], NULL);
    pthread_mutex_destroy(&J.lock);
    return J.failed ? -1 : 0;
}

int64_t orc_decode(const uint8_t *kpool, const uint8_t *vpool, int64_t num_blocks,
                   int64_t num_layers, int64_t block_size, int64_t num_kv_heads,
                   int64_t head_dim, int64_t dtype, int64_t layer, const uint8_t *q,
                   int64_t num_q_heads, const int32_t *block_tables, int64_t bt_stride,
                   const int32_t *seq_lens, const int32_t *offsets, int64_t num_seqs,
                   double scale, double *out, int64_t num_threads) {
    return run_attention(kpool, vpool, num_blocks, num_layers, block_size, num_kv_heads,
                         head_dim, dtype, layer, q, NULL, num_q_heads, block_tables, bt_stride,
                         seq_lens, offsets, num_seqs, scale, out, num_threads);
}

/* Prefill / append attention (see above): q_start[num_seqs + 1] are row
 * offsets into q and out, nondecreasing from q_start[0] = 0. */
int64_t orc_prefill(const uint8_t *kpool, const uint8_t *vpool, int64_t num_blocks,
                    int64_t num_layers, int64_t block_size, int64_t num_kv_heads,
                    int64_t head_dim, int64_t dtype, int64_t layer, const uint8_t *q,
                    const int32_t *q_start, int64_t num_q_heads, const int32_t *block_tables,
                    int64_t bt_stride, const int32_t *seq_lens, const int32_t *offsets,
                    int64_t num_seqs, double scale, double *out, int64_t num_threads) {
    if (!q_start || q_start[0] != 0) return -1;
    for (int64_t s = 0; s < num_seqs; s++)
        if (q_start[s + 1] < q_start[s]) return -1;
    return run_attention(kpool, vpool, num_blocks, num_layers, block_size, num_kv_heads,
                         head_dim, dtype, layer, q, q_start, num_q_heads, block_tables, bt_stride,
                         seq_lens, offsets, num_seqs, scale, out, num_threads);
}
