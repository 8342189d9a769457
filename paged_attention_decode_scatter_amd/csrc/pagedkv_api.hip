// pagedkv_api.hip -- the C ABI of libpagedkv.so (declared in pagedkv.h):
// host-side argument checks, launch geometry, dispatch to the kernels.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and needs no device.
#include <atomic>
#include <mutex>
#include <stdint.h>

#include "pagedkv.h"
#include "pkv_internal.h"

namespace {

using namespace pkv;

bool is_pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }

int ilog2(int64_t x) {
    int l = 0;
    while ((int64_t(1) << l) < x) ++l;
    return l;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t elem_bytes(int32_t dtype) { return dtype == PKV_BF16 ? 2 : dtype == PKV_I8 ? 1 : 4; }
bool is_quant(int32_t dtype) { return dtype == PKV_I8 || dtype == PKV_I4; }
// bits per code of a quantised pool
int quant_bits(int32_t dtype) { return dtype == PKV_I4 ? 4 : 8; }
// bytes of one token row (all kv heads) of one tensor
int64_t row_bytes_of(const pkv_pool *pool) {
    return pool->dtype == PKV_I4 ? pool->num_kv_heads * pool->head_dim / 2
                                 : pool->num_kv_heads * pool->head_dim * elem_bytes(pool->dtype);
}

int64_t pow2_or_neg(int64_t x) { return is_pow2(x) ? ilog2(x) : -1; }

// Common pool checks.  need_v: the call reads or writes V.
int check_pool(const pkv_pool *pool, bool need_v) {
    if (!pool) return PKV_ERR_NULL;
    if (pool->dtype != PKV_F32 && pool->dtype != PKV_BF16 && !is_quant(pool->dtype))
        return PKV_ERR_DTYPE;
    if (pool->reserved != 0) return PKV_ERR_SHAPE;
    if (pool->num_blocks <= 0 || pool->num_blocks > INT32_MAX || pool->num_layers <= 0 ||
        pool->num_kv_heads <= 0 || pool->head_dim <= 0 || !is_pow2(pool->block_size) ||
        pool->block_size > (1 << 20) || (pool->dtype == PKV_I4 && pool->head_dim % 2))
        return PKV_ERR_SHAPE;
    const int64_t row = row_bytes_of(pool);
    if (row > (int64_t(1) << 24)) return PKV_ERR_SHAPE;
    if (row % 16) return PKV_ERR_ALIGN;
    if (!pool->k || (need_v && !pool->v)) return PKV_ERR_NULL;
    if (!aligned16(pool->k) || (pool->v && !aligned16(pool->v))) return PKV_ERR_ALIGN;
    if (pool->block_stride != 0) {
        if (pool->block_stride < pool->num_layers * pool->block_size * row) return PKV_ERR_SHAPE;
        if (pool->block_stride % 16) return PKV_ERR_ALIGN;
    }
    if (is_quant(pool->dtype)) {
        if (!pool->k_scale || (pool->v && !pool->v_scale)) return PKV_ERR_NULL;
        if (!aligned16(pool->k_scale) || (pool->v && !aligned16(pool->v_scale)))
            return PKV_ERR_ALIGN;
    }
    return PKV_OK;
}

// Floats of one block's scales (all layers) in a quantised pool.
int64_t scale_block(const pkv_pool *pool) {
    return pool->num_layers * pool->num_kv_heads * pool->block_size;
}

// Bytes of one block of one tensor (all layers) and the distance between
// consecutive blocks.
int64_t dense_block_bytes(const pkv_pool *pool) {
    return pool->num_layers * pool->block_size * row_bytes_of(pool);
}
int64_t block_stride_of(const pkv_pool *pool) {
    return pool->block_stride ? pool->block_stride : dense_block_bytes(pool);
}

PoolView make_view(const pkv_pool *pool, int32_t layer) {
    PoolView v{};
    const int64_t row = row_bytes_of(pool);
    v.k = static_cast<const char *>(pool->k);
    v.v = static_cast<const char *>(pool->v);
    v.row_bytes = (int32_t)row;
    v.block_stride = block_stride_of(pool);
    v.layer_off = (int64_t)layer * pool->block_size * row;
    v.num_blocks = (int32_t)pool->num_blocks;
    v.lbs = ilog2(pool->block_size);
    if (is_quant(pool->dtype)) {
        const int64_t lo = (int64_t)layer * pool->num_kv_heads * pool->block_size;
        v.ks = static_cast<const float *>(pool->k_scale) + lo;
        v.vs = pool->v_scale ? static_cast<const float *>(pool->v_scale) + lo : nullptr;
        v.sc_block = scale_block(pool);
    }
    return v;
}

bool q8_dim_ok(const pkv_pool *pool) { return pool->head_dim == 64 || pool->head_dim == 128; }

// Compute units of the current device, queried once per device (256 when no
// device answers, e.g. on a build host).
int cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n > 0) return n;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cache[dev].store(n, std::memory_order_relaxed);
    return n;
}

// Largest split (multiple of 16 tokens) whose block-table entries fit the
// LDS staging buffer: ceil(S / bs) + 1 <= kBtLds.
int64_t max_split_tokens(int64_t bs) {
    int64_t s = (kBtLds - 2) * bs;
    if (s > (int64_t(1) << 20)) s = int64_t(1) << 20;
    return s - s % kChunkTokens;
}

bool split_ok(int64_t s, int64_t bs) {
    return s > 0 && s % kChunkTokens == 0 && s <= max_split_tokens(bs);
}

// Flat table positions a sequence of max_len tokens can span (its first
// block may start at any offset < bs).
int64_t max_positions(int64_t max_len, int64_t bs) { return max_len > 0 ? max_len + bs - 1 : 0; }

// Automatic split (a power of two >= 64 positions), from measured decode
// times on MI355X: grow the split while the work items (one wavefront each
// per (sequence, kv head, split) of max_seq_len tokens) exceed 8 per compute
// unit -- two resident workgroups of four -- and keep growing it up to 256
// positions while that still leaves at least 2 items per compute unit
// (shorter splits cost more per token in pipeline start-up and partials
// than they gain in balance).  Splits of 1024 positions and more keep
// growing while the items exceed 4 per compute unit (bf16 pools only): one
// resident workgroup per compute unit streaming twice as long measured
// faster (8 x 32768 tokens: 192.9 us at 2048 against 198.3 us at 1024, same
// process); the int8 kernel needs the second workgroup's wavefronts (141.6
// us at 2048 against 116 us at 1024).  With at least two (sequence, kv head)
// pairs per compute unit the bound is 32 items per compute unit instead and
// the long-split rule is off: such batches have many sequences of varied
// length, and shorter splits balance them (96 sequences of U[128, 4096]
// tokens, bf16: 172.0 us at 256, 162.9 at 512,
// 167.0 at 1024, 201.3 at 2048, 243.1 at 4096; 128 x U[128, 3072]: 158.2
// at 512, 185.7 at 2048; 256 x U[128, 1536]: level from 256 to 4096; int8,
// 96 x U[128, 4096]: 117.3 us at 512, 131.9 at 1024).  On the decode batch
// (32 x <= 2048 tokens) this picks 256; on 8 x 32768 tokens, 2048 for bf16,
// else 1024; on 96 x <= 4096 tokens, 512.  The split stops growing once it
// covers a whole sequence.
int64_t auto_split(int64_t num_seqs, int64_t hkv, int64_t max_len, int64_t bs, bool long_rule) {
    const int64_t cus = cu_count();
    const int64_t smax = max_split_tokens(bs);
    const int64_t span = max_positions(max_len, bs);
    const bool many = num_seqs * hkv >= 2 * cus;
    const int64_t per_cu = many ? 32 : 8;
    auto items = [&](int64_t s) { return num_seqs * hkv * ((max_len + s - 1) / s); };
    auto splits = [&](int64_t s) { return (span + s - 1) / s; };
    int64_t s = 64;
    if (s > smax) s = smax;
    while (s * 2 <= smax && s < span &&
           (items(s) > per_cu * cus || splits(s) > kMaxSplits || (s < 256 && items(s * 2) >= 2 * cus) ||
            (long_rule && !many && s >= 1024 && items(s) > 4 * cus)))
        s *= 2;
    return s;
}

struct DecodePlan {
    int64_t split;
    int64_t max_splits;
    int64_t cnt_bytes;  // per (sequence, head group) split counters, padded to 256 bytes
    int64_t ml_bytes;   // (m, l) partials, padded to 256 bytes
    int64_t acc_bytes;  // acc partials
    int64_t total() const { return cnt_bytes + ml_bytes + acc_bytes; }
};

int plan_decode(int64_t num_seqs, int64_t hkv, int64_t hq, int64_t head_dim, int64_t max_len,
                int64_t bs, int64_t split_req, DecodePlan *p, int32_t dtype = PKV_BF16) {
    if (num_seqs < 0 || hkv <= 0 || hq <= 0 || head_dim <= 0 || max_len < 0 || !is_pow2(bs))
        return PKV_ERR_SHAPE;
    // 0 (automatic) and a planned-schedule request plan the automatic
    // split too: it sizes the fallback and the workspace bound
    const int64_t split = split_req == 0 || split_req == PKV_SPLIT_PLANNED
                              ? auto_split(num_seqs, hkv, max_len, bs, dtype == PKV_BF16)
                              : split_req;
    if (!split_ok(split, bs)) return PKV_ERR_SHAPE;
    p->split = split;
    const int64_t span = max_positions(max_len, bs);
    p->max_splits = span > 0 ? (span + split - 1) / split : 1;
    if (p->max_splits > kMaxSplits) return PKV_ERR_SHAPE;
    if (p->max_splits <= 1) {
        p->max_splits = 1;
        p->cnt_bytes = p->ml_bytes = p->acc_bytes = 0;
    } else {
        // sized for one kv head per group, the most groups there can be
        p->cnt_bytes = (num_seqs * hkv * 4 + 255) / 256 * 256;
        const int64_t items = num_seqs * p->max_splits * hq;
        p->ml_bytes = (items * 2 * 4 + 255) / 256 * 256;
        p->acc_bytes = items * head_dim * 4;
    }
    return PKV_OK;
}

// kv heads (wavefronts) per decode workgroup: the largest of 4, 2, 1 that
// divides the kv head count.
int64_t heads_per_wg(int64_t hkv) {
    int64_t hpw = 1;
    while (hpw * 2 <= 4 && hkv % (hpw * 2) == 0) hpw *= 2;
    return hpw;
}

// Device-planned split schedule (bf16 and int8 pools): the grid is 2
// workgroups per compute unit (both resident: the bf16 decode kernel's LDS
// is about 55 KiB, the int8 one's 21 KiB; both use at most 256 registers),
// fewer when the pieces at the smallest split cannot fill it; each
// workgroup picks the split from the actual lengths (kernels_decode.hip).
// The smallest split keeps every sequence within 16 splits (merged in the
// kernel), and is at least 64 positions.  Possible when the grid holds 4
// pieces per (sequence, head group) -- so the device's split bound is at
// most max_len / 2 + 16 positions, which must fit the LDS table buffer --
// for at most kPlanMaxSeqs sequences, with positions below 2^24 (the
// kernel's float-reciprocal division).
struct SplitPlan {
    int64_t smin;
    int64_t wgs;
};

bool planned_possible(int64_t num_seqs, int64_t hkv, int64_t max_len, int64_t bs, int32_t dtype,
                      SplitPlan *sp) {
    if ((dtype != PKV_BF16 && !is_quant(dtype)) || num_seqs <= 0 || num_seqs > kPlanMaxSeqs || max_len <= 0 ||
        !is_pow2(bs))
        return false;
    const int64_t groups = hkv / heads_per_wg(hkv);
    const int64_t wgs_max = 2ll * cu_count();
    if (num_seqs * groups * 4 > wgs_max) return false;
    const int64_t span = max_positions(max_len, bs);
    if (span + bs >= (int64_t(1) << 24)) return false;
    const int64_t smax = max_split_tokens(bs);
    int64_t smin = ((span + 15) / 16 + 15) / 16 * 16;
    if (smin < 64) smin = 64;
    if (smin > smax || max_len / 2 + 32 > smax) return false;
    const int64_t max_splits = (span + smin - 1) / smin;
    const int64_t pieces_max = num_seqs * groups * max_splits;
    if (sp) {
        sp->smin = smin;
        sp->wgs = pieces_max < wgs_max ? pieces_max : wgs_max;
    }
    return true;
}

// Automatic (split_tokens = 0) and explicit (PKV_SPLIT_PLANNED) choice of
// the device-planned split.
bool use_planned(int64_t num_seqs, int64_t hkv, int64_t max_len, int64_t bs, int32_t dtype,
                 int64_t split_req, SplitPlan *sp) {
    if (split_req != 0 && split_req != PKV_SPLIT_PLANNED) return false;
    return planned_possible(num_seqs, hkv, max_len, bs, dtype, sp);
}

int status_of(hipError_t e) {
    if (e == hipSuccess) return PKV_OK;
    (void)hipGetLastError();
    return PKV_ERR_LAUNCH;
}

}  // namespace

extern "C" {

PKV_API int kv_slot_mapping(const int32_t *block_tables, int32_t bt_stride, const int32_t *offsets,
                            int32_t num_seqs, const int32_t *token_seq, const int32_t *token_pos,
                            int64_t num_tokens, int32_t block_size, int64_t *slot_mapping,
                            void *stream) {
    if (num_tokens < 0 || num_seqs < 0 || bt_stride < 0 || !is_pow2(block_size))
        return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!token_seq || !token_pos || !slot_mapping) return PKV_ERR_NULL;
    if (num_seqs > 0 && (!block_tables || !offsets)) return PKV_ERR_NULL;
    if (num_tokens > (int64_t(1) << 40)) return PKV_ERR_SHAPE;
    SlotArgs a{};
    a.block_tables = block_tables;
    a.offsets = offsets;
    a.token_seq = token_seq;
    a.token_pos = token_pos;
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.lbs = ilog2(block_size);
    return status_of(launch_slot_mapping(a, static_cast<hipStream_t>(stream)));
}

// Workgroup sizing shared by the scatter and the append: about 2048 16-byte
// pieces (32 KiB per tensor) per workgroup, but no fewer workgroups than a
// few per CU can absorb: a small scatter (one decode step's tokens) then
// runs one row per workgroup, each lane moving a single piece, so its
// latency is one load and one store.
static int64_t rows_per_wg(int64_t num_tokens, int64_t cpr) {
    int64_t tpw = 2048 / cpr;
    const int64_t wide = (num_tokens + 1023) / 1024;
    if (tpw > wide) tpw = wide;
    if (tpw < 1) tpw = 1;
    return tpw;
}

static ScatterQ8Args q8_args(const pkv_pool *pool, const PoolView &v, const void *k_src,
                             const void *v_src, int64_t num_tokens) {
    ScatterQ8Args a{};
    a.kpool = static_cast<char *>(pool->k);
    a.vpool = v_src ? static_cast<char *>(pool->v) : nullptr;
    a.ks = const_cast<float *>(v.ks);
    a.vs = v_src ? const_cast<float *>(v.vs) : nullptr;
    a.k_src = static_cast<const char *>(k_src);
    a.v_src = static_cast<const char *>(v_src);
    a.num_tokens = num_tokens;
    a.total_slots = pool->num_blocks * pool->block_size;
    a.block_stride = v.block_stride;
    a.layer_off = v.layer_off;
    a.sc_block = v.sc_block;
    a.num_kv_heads = (int32_t)pool->num_kv_heads;
    a.head_dim = (int32_t)pool->head_dim;
    a.lbs = v.lbs;
    a.qbits = quant_bits(pool->dtype);
    return a;
}

PKV_API int kv_scatter(const pkv_pool *pool, int32_t layer, const void *k_src, const void *v_src,
                       const int64_t *slot_mapping, int64_t num_tokens, void *stream) {
    const bool has_v = v_src != nullptr;
    int st = check_pool(pool, has_v);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_tokens < 0) return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_src || !slot_mapping) return PKV_ERR_NULL;
    if (!aligned16(k_src) || (has_v && !aligned16(v_src))) return PKV_ERR_ALIGN;
    const PoolView v = make_view(pool, layer);
    if (is_quant(pool->dtype)) {
        if (!q8_dim_ok(pool)) return PKV_ERR_UNSUPPORTED;
        if (num_tokens * pool->num_kv_heads > (int64_t)INT32_MAX * 8) return PKV_ERR_SHAPE;
        ScatterQ8Args a = q8_args(pool, v, k_src, v_src, num_tokens);
        a.slots = slot_mapping;
        return status_of(launch_scatter_q8(a, static_cast<hipStream_t>(stream)));
    }
    ScatterArgs a{};
    a.kpool = static_cast<char *>(pool->k);
    a.vpool = static_cast<char *>(pool->v);
    a.k_src = static_cast<const char *>(k_src);
    a.v_src = static_cast<const char *>(v_src);
    a.slots = slot_mapping;
    a.num_tokens = num_tokens;
    a.total_slots = pool->num_blocks * pool->block_size;
    a.block_stride = v.block_stride;
    a.layer_off = v.layer_off;
    a.row_bytes = v.row_bytes;
    a.lbs = v.lbs;
    const int64_t cpr = v.row_bytes / 16;
    const int64_t tpw = rows_per_wg(num_tokens, cpr);
    a.tok_per_wg = (int32_t)tpw;
    a.lcpr = (int32_t)pow2_or_neg(cpr);
    if (cpr * tpw > INT32_MAX / 2) return PKV_ERR_SHAPE;
    return status_of(launch_scatter(a, static_cast<hipStream_t>(stream)));
}

PKV_API int kv_append(const pkv_pool *pool, int32_t layer, const void *k_src, const void *v_src,
                      const int32_t *block_tables, int32_t bt_stride, const int32_t *offsets,
                      int32_t num_seqs, const int32_t *token_seq, const int32_t *token_pos,
                      int64_t num_tokens, int64_t *slot_mapping_out, void *stream) {
    const bool has_v = v_src != nullptr;
    int st = check_pool(pool, has_v);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_tokens < 0 || num_seqs < 0 || bt_stride < 0) return PKV_ERR_SHAPE;
    if (num_tokens == 0) return PKV_OK;
    if (!k_src || !token_seq || !token_pos || (num_seqs > 0 && (!block_tables || !offsets)))
        return PKV_ERR_NULL;
    if (!aligned16(k_src) || (has_v && !aligned16(v_src))) return PKV_ERR_ALIGN;
    const PoolView v = make_view(pool, layer);
    if (is_quant(pool->dtype)) {
        if (!q8_dim_ok(pool)) return PKV_ERR_UNSUPPORTED;
        if (num_tokens * pool->num_kv_heads > (int64_t)INT32_MAX * 8) return PKV_ERR_SHAPE;
        ScatterQ8Args a = q8_args(pool, v, k_src, v_src, num_tokens);
        a.block_tables = block_tables;
        a.offsets = offsets;
        a.token_seq = token_seq;
        a.token_pos = token_pos;
        a.slots_out = slot_mapping_out;
        a.bt_stride = bt_stride;
        a.num_seqs = num_seqs;
        return status_of(launch_scatter_q8(a, static_cast<hipStream_t>(stream)));
    }
    AppendArgs a{};
    a.sc.kpool = static_cast<char *>(pool->k);
    a.sc.vpool = static_cast<char *>(pool->v);
    a.sc.k_src = static_cast<const char *>(k_src);
    a.sc.v_src = static_cast<const char *>(v_src);
    a.sc.num_tokens = num_tokens;
    a.sc.total_slots = pool->num_blocks * pool->block_size;
    a.sc.block_stride = v.block_stride;
    a.sc.layer_off = v.layer_off;
    a.sc.row_bytes = v.row_bytes;
    a.sc.lbs = v.lbs;
    const int64_t cpr = v.row_bytes / 16;
    const int64_t tpw = rows_per_wg(num_tokens, cpr);
    a.sc.tok_per_wg = (int32_t)tpw;
    a.sc.lcpr = (int32_t)pow2_or_neg(cpr);
    if (cpr * tpw > INT32_MAX / 2) return PKV_ERR_SHAPE;
    a.block_tables = block_tables;
    a.offsets = offsets;
    a.token_seq = token_seq;
    a.token_pos = token_pos;
    a.slots_out = slot_mapping_out;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    return status_of(launch_append(a, static_cast<hipStream_t>(stream)));
}

PKV_API int kv_gather(const pkv_pool *pool, int32_t layer, const int32_t *block_tables,
                      int32_t bt_stride, const int32_t *seq_lens, const int32_t *offsets,
                      const int64_t *out_row_start, int32_t num_seqs, int32_t max_seq_len,
                      void *k_out, void *v_out, int64_t out_rows, void *stream) {
    const bool has_v = v_out != nullptr;
    int st = check_pool(pool, has_v);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_seqs < 0 || max_seq_len < 0 || bt_stride < 0 || out_rows < 0) return PKV_ERR_SHAPE;
    if (num_seqs == 0 || max_seq_len == 0 || out_rows == 0) return PKV_OK;
    if (!block_tables || !seq_lens || !offsets || !out_row_start || !k_out) return PKV_ERR_NULL;
    if (!aligned16(k_out) || (has_v && !aligned16(v_out))) return PKV_ERR_ALIGN;
    GatherArgs a{};
    a.pool = make_view(pool, layer);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.offsets = offsets;
    a.out_row_start = out_row_start;
    a.k_out = static_cast<char *>(k_out);
    a.v_out = static_cast<char *>(v_out);
    a.out_rows = out_rows;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    const int64_t cpr = a.pool.row_bytes / 16;
    int64_t tpw = 2048 / cpr;
    if (tpw < 1) tpw = 1;
    const int64_t tmax = (kBtLds - 2) * pool->block_size;  // LDS table capacity
    if (tpw > tmax) tpw = tmax;
    a.tok_per_wg = (int32_t)tpw;
    a.tiles_per_seq = (int32_t)((max_seq_len + tpw - 1) / tpw);
    a.lcpr = (int32_t)pow2_or_neg(cpr);
    if ((int64_t)num_seqs * a.tiles_per_seq > INT32_MAX || cpr * tpw > INT32_MAX / 2)
        return PKV_ERR_SHAPE;
    if (is_quant(pool->dtype)) {
        if (!q8_dim_ok(pool)) return PKV_ERR_UNSUPPORTED;
        return status_of(launch_gather_q8(a, (int)pool->head_dim, quant_bits(pool->dtype),
                                          static_cast<hipStream_t>(stream)));
    }
    return status_of(launch_gather(a, static_cast<hipStream_t>(stream)));
}

PKV_API int32_t paged_attn_decode_split_tokens(int32_t num_seqs, int32_t num_kv_heads,
                                               int32_t max_seq_len, int32_t block_size) {
    DecodePlan p;
    const int st = plan_decode(num_seqs, num_kv_heads, num_kv_heads, 64, max_seq_len, block_size,
                               0, &p);
    return st ? st : (int32_t)p.split;
}

PKV_API size_t paged_attn_decode_workspace_size(int32_t num_seqs, int32_t num_kv_heads,
                                                int32_t num_q_heads, int32_t head_dim,
                                                int32_t max_seq_len, int32_t block_size,
                                                int32_t split_tokens) {
    DecodePlan p, p8;
    if (num_kv_heads <= 0 || num_q_heads % num_kv_heads) return (size_t)-1;
    // the automatic split differs between bf16 and the other pool types:
    // room for either
    if (plan_decode(num_seqs, num_kv_heads, num_q_heads, head_dim, max_seq_len, block_size,
                    split_tokens, &p) ||
        plan_decode(num_seqs, num_kv_heads, num_q_heads, head_dim, max_seq_len, block_size,
                    split_tokens, &p8, PKV_I8))
        return (size_t)-1;
    int64_t need = p.total() > p8.total() ? p.total() : p8.total();
    SplitPlan sp2;
    if ((split_tokens == 0 || split_tokens == PKV_SPLIT_PLANNED) &&
        planned_possible(num_seqs, num_kv_heads, max_seq_len, block_size, PKV_BF16, &sp2)) {
        DecodePlan pp;
        if (plan_decode(num_seqs, num_kv_heads, num_q_heads, head_dim, max_seq_len, block_size,
                        sp2.smin, &pp))
            return (size_t)-1;
        if (pp.total() > need) need = pp.total();
    }
    return (size_t)need;
}

PKV_API int32_t paged_attn_decode_schedule(int32_t num_seqs, int32_t num_kv_heads,
                                           int32_t num_q_heads, int32_t head_dim,
                                           int32_t max_seq_len, int32_t block_size, int32_t dtype,
                                           int32_t split_tokens) {
    if (dtype != PKV_F32 && dtype != PKV_BF16 && !is_quant(dtype)) return PKV_ERR_DTYPE;
    if (num_kv_heads <= 0 || num_q_heads <= 0 || num_q_heads % num_kv_heads) return PKV_ERR_SHAPE;
    DecodePlan p;
    const int st = plan_decode(num_seqs, num_kv_heads, num_q_heads, head_dim, max_seq_len,
                               block_size, split_tokens, &p, dtype);
    if (st) return st;
    if (use_planned(num_seqs, num_kv_heads, max_seq_len, block_size, dtype, split_tokens, nullptr))
        return PKV_SCHEDULE_PLANNED;
    if (split_tokens == PKV_SPLIT_PLANNED) return PKV_ERR_UNSUPPORTED;
    return (int32_t)p.split;
}

}  // extern "C"

namespace {

// paged_attn_decode, and paged_attn_decode_append when k_new is given.
// clear_cnt: zero the workspace's merge counters (a fill kernel on the
// stream) before the decode, for a workspace whose earlier contents are not
// known to be clean.
int decode_impl(const pkv_pool *pool, int32_t layer, const void *q, int32_t num_q_heads,
                const void *k_new, const void *v_new, const int32_t *block_tables, int32_t bt_stride,
                const int32_t *seq_lens, const int32_t *offsets, int32_t num_seqs,
                int32_t max_seq_len, float scale, int32_t split_tokens, void *out,
                void *workspace, size_t workspace_bytes, void *stream, bool clear_cnt = false) {
    int st = check_pool(pool, true);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_seqs < 0 || max_seq_len < 0 || bt_stride < 0 || num_q_heads <= 0 ||
        num_q_heads % pool->num_kv_heads != 0 ||
        (split_tokens < 0 && split_tokens != PKV_SPLIT_PLANNED))
        return PKV_ERR_SHAPE;
    const int group = (int)(num_q_heads / pool->num_kv_heads);
    if (!decode_supported(pool->dtype, (int)pool->head_dim, group)) return PKV_ERR_UNSUPPORTED;
    SplitPlan spl{};
    const bool planned = use_planned(num_seqs, pool->num_kv_heads, max_seq_len, pool->block_size,
                                     pool->dtype, split_tokens, &spl);
    if (split_tokens == PKV_SPLIT_PLANNED && !planned) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PKV_OK;
    if (!q || !out || !seq_lens || !offsets || (max_seq_len > 0 && !block_tables))
        return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return PKV_ERR_ALIGN;
    if (k_new && !v_new) return PKV_ERR_NULL;
    if (k_new && (!aligned16(k_new) || !aligned16(v_new))) return PKV_ERR_ALIGN;
    DecodePlan p;
    st = plan_decode(num_seqs, pool->num_kv_heads, num_q_heads, pool->head_dim, max_seq_len,
                     pool->block_size, planned ? (int32_t)spl.smin : split_tokens, &p, pool->dtype);
    if (st) return st;
    const int64_t need = p.total();
    if (need > 0) {
        if (!workspace || (int64_t)workspace_bytes < need) return PKV_ERR_WORKSPACE;
        if (!aligned16(workspace)) return PKV_ERR_ALIGN;
    }
    const int64_t hkv = pool->num_kv_heads;
    const int64_t hpw = heads_per_wg(hkv);
    const int64_t groups = hkv / hpw;
    if (groups * p.max_splits * num_seqs > INT32_MAX) return PKV_ERR_SHAPE;
    DecodeArgs a{};
    a.pool = make_view(pool, layer);
    a.q = static_cast<const char *>(q);
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.offsets = offsets;
    a.out = static_cast<char *>(out);
    a.k_new = static_cast<const char *>(k_new);
    a.v_new = static_cast<const char *>(v_new);
    char *ws = need > 0 ? static_cast<char *>(workspace) : nullptr;
    const int64_t cnt_bytes = p.cnt_bytes;
    const int64_t ml_bytes = p.ml_bytes;
    a.ws_cnt = ws ? reinterpret_cast<uint32_t *>(ws) : nullptr;
    a.ws_ml = ws ? reinterpret_cast<float *>(ws + cnt_bytes) : nullptr;
    a.ws_acc = ws ? reinterpret_cast<float *>(ws + cnt_bytes + ml_bytes) : nullptr;
    a.scale_log2 = scale * 1.4426950408889634f;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.num_kv_heads = (int32_t)hkv;
    a.num_q_heads = num_q_heads;
    a.split_tokens = (int32_t)p.split;
    a.max_splits = (int32_t)p.max_splits;
    a.heads_per_wg = (int32_t)hpw;
    a.head_groups = (int32_t)groups;
    a.fused_merge = p.max_splits <= kFusedMergeMaxSplits;
    a.plan = planned ? (int32_t)spl.wgs : 0;
    a.max_len = max_seq_len;
    if (clear_cnt && ws && cnt_bytes > 0) {
        const hipError_t e = launch_zero_words(a.ws_cnt, cnt_bytes / 4, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return status_of(e);
    }
    if (k_new && is_quant(pool->dtype)) {
        // quantised pool: the new rows are quantised and written by the
        // append kernel in decode-step mode, then decode runs over the pool
        // (two launches on the stream; the row's quantisation needs the
        // whole row, which the attention kernel's work item does not hold)
        ScatterQ8Args w = q8_args(pool, a.pool, k_new, v_new, num_seqs);
        w.block_tables = block_tables;
        w.offsets = offsets;
        w.step_lens = seq_lens;
        w.step_max_len = max_seq_len;
        w.bt_stride = bt_stride;
        w.num_seqs = num_seqs;
        const hipError_t e = launch_scatter_q8(w, static_cast<hipStream_t>(stream));
        if (e != hipSuccess) return status_of(e);
        a.k_new = nullptr;
        a.v_new = nullptr;
    }
    return status_of(launch_decode(a, pool->dtype, (int)pool->head_dim, group,
                                   static_cast<hipStream_t>(stream)));
}

// The fixed device scratch of paged_attn_decode_noalloc: the split
// partials and merge counters of every call on a device live here (each
// device holds its own copy for the life of the process; zero when the
// code object is loaded).  Host code never passes the array's name to a
// kernel: its device address is looked up once per device below.
static __device__ __align__(256) unsigned char scratch[PKV_NOALLOC_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up with that
// device current on the first call and kept per device; nullptr if the
// lookup fails.
char *scratch_ptr() {
    constexpr int kMaxDev = 64;
    static std::atomic<char *> cache[kMaxDev];
    static std::mutex mu;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
        (void)hipGetLastError();
        return nullptr;
    }
    char *p = cache[dev].load(std::memory_order_acquire);
    if (p) return p;
    std::lock_guard<std::mutex> lock(mu);
    p = cache[dev].load(std::memory_order_relaxed);
    if (p) return p;
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        (void)hipGetLastError();
        return nullptr;
    }
    p = static_cast<char *>(addr);
    cache[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

PKV_API int paged_attn_decode(const pkv_pool *pool, int32_t layer, const void *q,
                              int32_t num_q_heads, const int32_t *block_tables, int32_t bt_stride,
                              const int32_t *seq_lens, const int32_t *offsets, int32_t num_seqs,
                              int32_t max_seq_len, float scale, int32_t split_tokens, void *out,
                              void *workspace, size_t workspace_bytes, void *stream) {
    return decode_impl(pool, layer, q, num_q_heads, nullptr, nullptr, block_tables, bt_stride,
                       seq_lens, offsets, num_seqs, max_seq_len, scale, split_tokens, out, workspace,
                       workspace_bytes, stream);
}

PKV_API int paged_attn_decode_noalloc(const pkv_pool *pool, int32_t layer, const void *q,
                                      int32_t num_q_heads, const int32_t *block_tables,
                                      int32_t bt_stride, const int32_t *seq_lens,
                                      const int32_t *offsets, int32_t num_seqs, int32_t max_seq_len,
                                      float scale, int32_t split_tokens, void *out, void *stream) {
    int st = check_pool(pool, true);
    if (st) return st;
    if (num_seqs < 0 || max_seq_len < 0 || num_q_heads <= 0 || num_q_heads % pool->num_kv_heads)
        return PKV_ERR_SHAPE;
    const size_t need = paged_attn_decode_workspace_size(
        num_seqs, (int32_t)pool->num_kv_heads, num_q_heads, (int32_t)pool->head_dim, max_seq_len,
        (int32_t)pool->block_size, split_tokens);
    if (need == (size_t)-1) return PKV_ERR_SHAPE;
    if (need > (size_t)PKV_NOALLOC_SCRATCH_BYTES) return PKV_ERR_SCRATCH;
    char *ws = nullptr;
    if (need > 0 && num_seqs > 0) {
        ws = scratch_ptr();
        if (!ws) return PKV_ERR_DEVICE;
    }
    return decode_impl(pool, layer, q, num_q_heads, nullptr, nullptr, block_tables, bt_stride,
                       seq_lens, offsets, num_seqs, max_seq_len, scale, split_tokens, out, ws,
                       ws ? (size_t)PKV_NOALLOC_SCRATCH_BYTES : 0, stream, /*clear_cnt=*/true);
}

PKV_API int paged_attn_decode_append(const pkv_pool *pool, int32_t layer, const void *q,
                                     int32_t num_q_heads, const void *k_new, const void *v_new,
                                     const int32_t *block_tables, int32_t bt_stride,
                                     const int32_t *seq_lens, const int32_t *offsets,
                                     int32_t num_seqs, int32_t max_seq_len, float scale,
                                     int32_t split_tokens, void *out, void *workspace,
                                     size_t workspace_bytes, void *stream) {
    if (num_seqs > 0 && (!k_new || !v_new)) return PKV_ERR_NULL;
    return decode_impl(pool, layer, q, num_q_heads, k_new, v_new, block_tables, bt_stride, seq_lens,
                       offsets, num_seqs, max_seq_len, scale, split_tokens, out, workspace,
                       workspace_bytes, stream);
}

PKV_API int paged_attn_prefill(const pkv_pool *pool, int32_t layer, const void *q,
                               int32_t num_q_heads, const int32_t *q_start, int32_t num_q_rows,
                               int32_t max_q_len, const int32_t *block_tables, int32_t bt_stride,
                               const int32_t *seq_lens, const int32_t *offsets, int32_t num_seqs,
                               float scale, void *out, void *stream) {
    int st = check_pool(pool, true);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_seqs < 0 || num_q_rows < 0 || max_q_len < 0 || bt_stride < 0 || num_q_heads <= 0 ||
        num_q_heads % pool->num_kv_heads != 0)
        return PKV_ERR_SHAPE;
    const int group = (int)(num_q_heads / pool->num_kv_heads);
    if (!prefill_supported(pool->dtype, (int)pool->head_dim, group)) return PKV_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_q_rows == 0) return PKV_OK;
    if (!q || !out || !q_start || !seq_lens || !offsets || !block_tables) return PKV_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return PKV_ERR_ALIGN;
    const int64_t hkv = pool->num_kv_heads;
    const int64_t hpw = heads_per_wg(hkv);
    const int64_t tile = pool->dtype == PKV_BF16 ? prefill_tile(pool->head_dim, group) : 16;
    const int64_t q_tiles = ((int64_t)max_q_len + tile - 1) / tile;
    if (q_tiles * num_seqs * hkv > INT32_MAX || (int64_t)num_q_rows * (hkv / hpw) > INT32_MAX)
        return PKV_ERR_SHAPE;
    if (q_tiles == 0) return PKV_OK;
    PrefillArgs a{};
    a.pool = make_view(pool, layer);
    a.q = static_cast<const char *>(q);
    a.q_start = q_start;
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.offsets = offsets;
    a.out = static_cast<char *>(out);
    a.scale_log2 = scale * 1.4426950408889634f;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.num_kv_heads = (int32_t)hkv;
    a.num_q_heads = num_q_heads;
    a.num_q_rows = num_q_rows;
    a.q_tiles = (int32_t)q_tiles;
    a.max_q_len = max_q_len;
    a.heads_per_wg = (int32_t)hpw;
    a.head_groups = (int32_t)(hkv / hpw);
    a.seg_chunks = (int32_t)(max_split_tokens(pool->block_size) / kChunkTokens);
    return status_of(launch_prefill(a, pool->dtype, (int)pool->head_dim, group,
                                    static_cast<hipStream_t>(stream)));
}

PKV_API int kv_read_blocks(const pkv_pool *pool, int32_t layer, const int32_t *block_ids,
                           int64_t num_ids, uint32_t *out, void *stream) {
    int st = check_pool(pool, false);
    if (st) return st;
    if (layer < 0 || layer >= pool->num_layers) return PKV_ERR_LAYER;
    if (num_ids < 0 || num_ids > INT32_MAX) return PKV_ERR_SHAPE;
    if (num_ids == 0) return PKV_OK;
    if (!block_ids || !out) return PKV_ERR_NULL;
    const PoolView v = make_view(pool, layer);
    ReadBlocksArgs a{};
    a.k = v.k;
    a.v = v.v;
    a.ids = block_ids;
    a.out = out;
    a.n = num_ids;
    a.num_blocks = pool->num_blocks;
    a.block_stride = v.block_stride;
    a.layer_off = v.layer_off;
    a.slice_bytes = (int64_t)v.row_bytes << v.lbs;
    return status_of(launch_read_blocks(a, static_cast<hipStream_t>(stream)));
}

PKV_API int kv_copy_blocks(const pkv_pool *pool, const int32_t *src_blocks,
                           const int32_t *dst_blocks, int64_t num_pairs, void *stream) {
    int st = check_pool(pool, false);
    if (st) return st;
    if (num_pairs < 0) return PKV_ERR_SHAPE;
    if (num_pairs == 0) return PKV_OK;
    if (!src_blocks || !dst_blocks) return PKV_ERR_NULL;
    CopyBlocksArgs a{};
    a.k = static_cast<char *>(pool->k);
    a.v = static_cast<char *>(pool->v);
    a.src = src_blocks;
    a.dst = dst_blocks;
    a.num_pairs = num_pairs;
    a.num_blocks = pool->num_blocks;
    a.block_bytes = dense_block_bytes(pool);
    a.block_stride = block_stride_of(pool);
    a.pieces = (a.block_bytes + kCopyBlockPiece - 1) / kCopyBlockPiece;
    if (a.pieces * num_pairs > INT32_MAX) return PKV_ERR_SHAPE;
    st = status_of(launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
    if (st || !is_quant(pool->dtype)) return st;
    // the scales of a quantised pool: one dense range per block as well
    a.k = static_cast<char *>(pool->k_scale);
    a.v = pool->v ? static_cast<char *>(pool->v_scale) : nullptr;
    a.block_bytes = a.block_stride = scale_block(pool) * 4;
    a.pieces = (a.block_bytes + kCopyBlockPiece - 1) / kCopyBlockPiece;
    return status_of(launch_copy_blocks(a, static_cast<hipStream_t>(stream)));
}

namespace {

// Host <-> pool block moves: runs of consecutive ids in a dense pool as one
// copy each.
int swap_impl(const pkv_pool *pool, const int32_t *ids, int64_t n, char *kh, char *vh,
              bool to_host, void *stream) {
    int st = check_pool(pool, false);
    if (st) return st;
    if (n < 0) return PKV_ERR_SHAPE;
    if (n == 0) return PKV_OK;
    if (!ids || !kh || (pool->v && !vh)) return PKV_ERR_NULL;
    for (int64_t i = 0; i < n; ++i)
        if (ids[i] < 0 || ids[i] >= pool->num_blocks) return PKV_ERR_BLOCK;
    const int64_t bb = dense_block_bytes(pool);
    const int64_t stride = block_stride_of(pool);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const hipMemcpyKind kind = to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
    for (int64_t i = 0; i < n;) {
        int64_t j = i + 1;
        while (stride == bb && j < n && ids[j] == ids[j - 1] + 1) ++j;
        const int64_t bytes = (j - i) * bb;
        for (int t = 0; t < 2; ++t) {
            char *dev = static_cast<char *>(t == 0 ? pool->k : pool->v);
            char *host = t == 0 ? kh : vh;
            if (!dev) continue;
            char *d = dev + (int64_t)ids[i] * stride;
            char *h = host + i * bb;
            const hipError_t e = to_host ? hipMemcpyAsync(h, d, bytes, kind, s)
                                         : hipMemcpyAsync(d, h, bytes, kind, s);
            if (e != hipSuccess) return status_of(e);
        }
        i = j;
    }
    if (!is_quant(pool->dtype)) return PKV_OK;
    // quantised pool: the n blocks' scales follow the n blocks' codes
    const int64_t sb = scale_block(pool) * 4;
    for (int64_t i = 0; i < n;) {
        int64_t j = i + 1;
        while (j < n && ids[j] == ids[j - 1] + 1) ++j;
        for (int t = 0; t < 2; ++t) {
            char *dev = static_cast<char *>(t == 0 ? pool->k_scale : (pool->v ? pool->v_scale : nullptr));
            char *host = t == 0 ? kh : vh;
            if (!dev) continue;
            char *d = dev + (int64_t)ids[i] * sb;
            char *h = host + n * bb + i * sb;
            const hipError_t e = to_host ? hipMemcpyAsync(h, d, (j - i) * sb, kind, s)
                                         : hipMemcpyAsync(d, h, (j - i) * sb, kind, s);
            if (e != hipSuccess) return status_of(e);
        }
        i = j;
    }
    return PKV_OK;
}

}  // namespace

PKV_API int kv_swap_out(const pkv_pool *pool, const int32_t *block_ids, int64_t n, void *k_host,
                        void *v_host, void *stream) {
    return swap_impl(pool, block_ids, n, static_cast<char *>(k_host), static_cast<char *>(v_host),
                     true, stream);
}

PKV_API int kv_swap_in(const pkv_pool *pool, const int32_t *block_ids, int64_t n,
                       const void *k_host, const void *v_host, void *stream) {
    return swap_impl(pool, block_ids, n, static_cast<char *>(const_cast<void *>(k_host)),
                     static_cast<char *>(const_cast<void *>(v_host)), false, stream);
}

PKV_API int kv_validate(const pkv_pool *pool, const int32_t *block_tables, int32_t bt_stride,
                        const int32_t *seq_lens, const int32_t *offsets, int32_t num_seqs,
                        int32_t max_seq_len, const int64_t *slot_mapping, int64_t num_tokens,
                        int64_t *violations, void *stream) {
    if (!pool || !violations) return PKV_ERR_NULL;
    if (pool->num_blocks <= 0 || pool->num_blocks > INT32_MAX || !is_pow2(pool->block_size))
        return PKV_ERR_SHAPE;
    if (num_seqs < 0 || bt_stride < 0 || num_tokens < 0) return PKV_ERR_SHAPE;
    if (num_seqs > 0 && (!block_tables || !seq_lens || !offsets)) return PKV_ERR_NULL;
    if (num_tokens > 0 && !slot_mapping) return PKV_ERR_NULL;
    ValidateArgs a{};
    a.block_tables = block_tables;
    a.seq_lens = seq_lens;
    a.offsets = offsets;
    a.slots = slot_mapping;
    a.count = reinterpret_cast<unsigned long long *>(violations);
    a.num_tokens = num_tokens;
    a.total_slots = pool->num_blocks * pool->block_size;
    a.bt_stride = bt_stride;
    a.num_seqs = num_seqs;
    a.num_blocks = (int32_t)pool->num_blocks;
    a.block_size = (int32_t)pool->block_size;
    a.max_seq_len = max_seq_len;
    return status_of(launch_validate(a, static_cast<hipStream_t>(stream)));
}

PKV_API const char *pkv_status_string(int status) {
    switch (status) {
        case PKV_OK: return "ok";
        case PKV_ERR_NULL: return "a required pointer is NULL";
        case PKV_ERR_DTYPE: return "unknown element type";
        case PKV_ERR_SHAPE: return "invalid size or shape";
        case PKV_ERR_LAYER: return "layer outside [0, num_layers)";
        case PKV_ERR_ALIGN: return "pointer or row not 16-byte aligned";
        case PKV_ERR_WORKSPACE: return "workspace missing or too small";
        case PKV_ERR_LAUNCH: return "HIP kernel launch failed";
        case PKV_ERR_UNSUPPORTED: return "head_dim or query-group size not supported";
        case PKV_ERR_DEVICE: return "no usable HIP device";
        case PKV_ERR_SEQ: return "unknown or duplicate sequence id";
        case PKV_ERR_BLOCK: return "block id out of range or free";
        case PKV_ERR_HOST: return "host memory could not be allocated";
        case PKV_ERR_SCRATCH:
            return "the decode workspace these sizes need exceeds the fixed device scratch "
                   "(PKV_NOALLOC_SCRATCH_BYTES)";
        case PKV_NO_SPACE: return "too few free blocks (nothing changed)";
        default: return "unknown status";
    }
}

}  // extern "C"
