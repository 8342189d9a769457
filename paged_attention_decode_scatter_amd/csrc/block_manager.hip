// block_manager.hip -- host-side block manager (no device code): FIFO free
// queue of physical block ids, per-block reference counts and per-sequence
// block tables with a first-block offset, after [P2 sec. 2.1] and
// [P3 secs. 2.2-2.4] ("vLLM PagedAttention source notes"; mini-runtime
// ch. 12 "Paged KV Cache").  Every entry point checks its arguments first
// and changes nothing on an error; host allocation failures (only possible
// where a table or the sequence map grows) are caught before any block is
// taken and reported as PKV_ERR_HOST.
#include <cstdint>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_block_manager.h"

struct pkv_block_manager {
    struct Seq {
        std::vector<int32_t> blocks;  // physical ids in logical order
        int32_t offset = 0;           // first-block start position
        int64_t len = 0;              // tokens held
    };
    // FIFO of free ids as a ring of num_blocks entries: a block is in it
    // exactly when its count is 0, so it never holds more, and pushing never
    // allocates (freeing cannot fail half-way).
    struct Ring {
        std::vector<int32_t> q;
        int64_t head = 0, count = 0;
        int64_t size() const { return count; }
        bool empty() const { return count == 0; }
        int32_t front() const { return q[head]; }
        void pop_front() {
            head = head + 1 == (int64_t)q.size() ? 0 : head + 1;
            --count;
        }
        void push_back(int32_t b) {
            int64_t i = head + count;
            if (i >= (int64_t)q.size()) i -= (int64_t)q.size();
            q[i] = b;
            ++count;
        }
        int32_t at(int64_t i) const {
            int64_t k = head + i;
            if (k >= (int64_t)q.size()) k -= (int64_t)q.size();
            return q[k];
        }
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::vector<int32_t> ref;         // reference count per block (0 = free)
    Ring free_q;                      // free ids, front = next to hand out
    std::unordered_map<int64_t, Seq> seqs;
    int64_t peak_used = 0;

    int64_t used() const { return (int64_t)num_blocks - free_q.size(); }
    void note_peak() {
        if (used() > peak_used) peak_used = used();
    }
    // blocks a sequence of n tokens from flat position `offset` needs
    int64_t blocks_for(int64_t n, int64_t offset) const {
        return n > 0 ? (offset + n + block_size - 1) / block_size : 0;
    }
    Seq *find(int64_t seq) {
        auto it = seqs.find(seq);
        return it == seqs.end() ? nullptr : &it->second;
    }
    const Seq *find(int64_t seq) const {
        auto it = seqs.find(seq);
        return it == seqs.end() ? nullptr : &it->second;
    }
    int32_t take() {  // caller checked the queue is not empty
        const int32_t b = free_q.front();
        free_q.pop_front();
        ref[b] = 1;
        return b;
    }
    void drop(int32_t b) {  // one reference less; 0 -> back of the queue
        if (--ref[b] == 0) free_q.push_back(b);
    }
};

namespace {

// Run f, turning a host allocation failure into PKV_ERR_HOST.
template <typename F>
int guarded(F &&f) {
    try {
        return f();
    } catch (const std::bad_alloc &) {
        return PKV_ERR_HOST;
    }
}

}  // namespace

extern "C" {

PKV_API pkv_block_manager *pkv_bm_create(int32_t num_blocks, int32_t block_size) {
    if (num_blocks <= 0 || block_size <= 0) return nullptr;
    try {
        auto *bm = new pkv_block_manager();
        bm->num_blocks = num_blocks;
        bm->block_size = block_size;
        bm->ref.assign(num_blocks, 0);
        bm->free_q.q.assign(num_blocks, 0);
        for (int32_t b = 0; b < num_blocks; ++b) bm->free_q.push_back(b);
        return bm;
    } catch (const std::bad_alloc &) {
        return nullptr;
    }
}

PKV_API void pkv_bm_destroy(pkv_block_manager *bm) { delete bm; }

PKV_API int pkv_bm_can_allocate(const pkv_block_manager *bm, int64_t num_tokens, int32_t offset) {
    if (!bm) return PKV_ERR_NULL;
    if (num_tokens < 0 || offset < 0 || offset >= bm->block_size) return PKV_ERR_SHAPE;
    return bm->blocks_for(num_tokens, offset) <= bm->free_q.size() ? 1 : 0;
}

PKV_API int pkv_bm_allocate(pkv_block_manager *bm, int64_t seq, int64_t num_tokens, int32_t offset) {
    if (!bm) return PKV_ERR_NULL;
    if (num_tokens < 0 || offset < 0 || offset >= bm->block_size) return PKV_ERR_SHAPE;
    if (bm->find(seq)) return PKV_ERR_SEQ;
    const int64_t need = bm->blocks_for(num_tokens, offset);
    if (need > bm->free_q.size()) return PKV_NO_SPACE;
    return guarded([&] {
        pkv_block_manager::Seq s;
        s.blocks.reserve(need);
        s.offset = offset;
        s.len = num_tokens;
        auto &slot = bm->seqs[seq];  // may throw: nothing taken yet
        for (int64_t i = 0; i < need; ++i) s.blocks.push_back(bm->take());
        slot = std::move(s);
        bm->note_peak();
        return PKV_OK;
    });
}

PKV_API int pkv_bm_share(pkv_block_manager *bm, int64_t src, int64_t dst, int32_t num_blocks) {
    if (!bm) return PKV_ERR_NULL;
    const pkv_block_manager::Seq *s = bm->find(src);
    if (!s || bm->find(dst)) return PKV_ERR_SEQ;
    if (num_blocks < 1 || num_blocks > (int64_t)s->blocks.size()) return PKV_ERR_SHAPE;
    return guarded([&] {
        pkv_block_manager::Seq d;
        d.blocks.assign(s->blocks.begin(), s->blocks.begin() + num_blocks);
        d.offset = s->offset;
        d.len = (int64_t)num_blocks * bm->block_size - s->offset;
        bm->seqs.emplace(dst, std::move(d));  // may throw: no count changed yet
        for (int32_t i = 0; i < num_blocks; ++i) ++bm->ref[bm->seqs[dst].blocks[i]];
        return PKV_OK;
    });
}

PKV_API int pkv_bm_append_slot(pkv_block_manager *bm, int64_t seq, int64_t *slot) {
    if (!bm || !slot) return PKV_ERR_NULL;
    pkv_block_manager::Seq *s = bm->find(seq);
    if (!s) return PKV_ERR_SEQ;
    const int64_t p = s->offset + s->len;
    const int64_t j = p / bm->block_size;
    const int64_t k = p % bm->block_size;
    if (j == (int64_t)s->blocks.size()) {
        if (bm->free_q.empty()) return PKV_NO_SPACE;
        const int st = guarded([&] {
            s->blocks.reserve(s->blocks.size() + 1);  // may throw before anything is taken
            s->blocks.push_back(bm->take());
            return PKV_OK;
        });
        if (st) return st;
        bm->note_peak();
    }
    s->len += 1;
    *slot = (int64_t)s->blocks[j] * bm->block_size + k;
    return PKV_OK;
}

PKV_API int32_t pkv_bm_append_slots(pkv_block_manager *bm, const int64_t *seqs, int32_t n,
                                    int64_t *slots) {
    if (!bm || (n > 0 && (!seqs || !slots))) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    for (int32_t i = 0; i < n; ++i)
        if (!bm->find(seqs[i])) return PKV_ERR_SEQ;
    for (int32_t i = 0; i < n; ++i) {
        if (pkv_bm_append_slot(bm, seqs[i], &slots[i]) != PKV_OK) return i;
    }
    return n;
}

PKV_API int pkv_bm_free(pkv_block_manager *bm, int64_t seq) {
    if (!bm) return PKV_ERR_NULL;
    auto it = bm->seqs.find(seq);
    if (it == bm->seqs.end()) return PKV_ERR_SEQ;
    for (int32_t b : it->second.blocks) bm->drop(b);
    bm->seqs.erase(it);
    return PKV_OK;
}

PKV_API int pkv_bm_cow(pkv_block_manager *bm, int64_t seq, int32_t index, int32_t *src_block,
                       int32_t *dst_block) {
    if (!bm || !src_block || !dst_block) return PKV_ERR_NULL;
    pkv_block_manager::Seq *s = bm->find(seq);
    if (!s) return PKV_ERR_SEQ;
    if (index < 0 || index >= (int64_t)s->blocks.size()) return PKV_ERR_SHAPE;
    const int32_t b = s->blocks[index];
    if (bm->ref[b] <= 1) {  // unshared: written in place
        *src_block = *dst_block = b;
        return PKV_OK;
    }
    if (bm->free_q.empty()) return PKV_NO_SPACE;
    const int32_t nb = bm->take();
    s->blocks[index] = nb;
    bm->drop(b);  // still held by the other tables: stays out of the queue
    bm->note_peak();
    *src_block = b;
    *dst_block = nb;
    return PKV_OK;
}

PKV_API int pkv_bm_inc_ref(pkv_block_manager *bm, int32_t block) {
    if (!bm) return PKV_ERR_NULL;
    if (block < 0 || block >= bm->num_blocks || bm->ref[block] <= 0) return PKV_ERR_BLOCK;
    ++bm->ref[block];
    return PKV_OK;
}

PKV_API int pkv_bm_dec_ref(pkv_block_manager *bm, int32_t block) {
    if (!bm) return PKV_ERR_NULL;
    if (block < 0 || block >= bm->num_blocks || bm->ref[block] <= 0) return PKV_ERR_BLOCK;
    bm->drop(block);
    return PKV_OK;
}

PKV_API int64_t pkv_bm_seq_len(const pkv_block_manager *bm, int64_t seq) {
    if (!bm) return PKV_ERR_NULL;
    const pkv_block_manager::Seq *s = bm->find(seq);
    return s ? s->len : PKV_ERR_SEQ;
}

PKV_API int32_t pkv_bm_max_blocks(const pkv_block_manager *bm, const int64_t *seqs, int32_t n) {
    if (!bm || (n > 0 && !seqs)) return PKV_ERR_NULL;
    if (n < 0) return PKV_ERR_SHAPE;
    int32_t m = 0;
    for (int32_t i = 0; i < n; ++i) {
        const pkv_block_manager::Seq *s = bm->find(seqs[i]);
        if (!s) return PKV_ERR_SEQ;
        if ((int32_t)s->blocks.size() > m) m = (int32_t)s->blocks.size();
    }
    return m;
}

PKV_API int pkv_bm_tables(const pkv_block_manager *bm, const int64_t *seqs, int32_t n,
                          int32_t *tables, int32_t stride, int32_t *seq_lens, int32_t *offsets) {
    if (!bm || (n > 0 && (!seqs || (!tables && stride > 0)))) return PKV_ERR_NULL;
    if (n < 0 || stride < 0) return PKV_ERR_SHAPE;
    for (int32_t i = 0; i < n; ++i) {
        const pkv_block_manager::Seq *s = bm->find(seqs[i]);
        if (!s) return PKV_ERR_SEQ;
        if ((int64_t)s->blocks.size() > stride || s->len > INT32_MAX) return PKV_ERR_SHAPE;
    }
    for (int32_t i = 0; i < n; ++i) {
        const pkv_block_manager::Seq *s = bm->find(seqs[i]);
        int32_t *row = tables + (int64_t)i * stride;
        const int32_t nb = (int32_t)s->blocks.size();
        for (int32_t j = 0; j < stride; ++j) row[j] = j < nb ? s->blocks[j] : -1;
        if (seq_lens) seq_lens[i] = (int32_t)s->len;
        if (offsets) offsets[i] = s->offset;
    }
    return PKV_OK;
}

PKV_API int32_t pkv_bm_free_queue(const pkv_block_manager *bm, int32_t *ids, int32_t cap) {
    if (!bm || (cap > 0 && !ids)) return PKV_ERR_NULL;
    for (int64_t i = 0; i < cap && i < bm->free_q.size(); ++i) ids[i] = bm->free_q.at(i);
    return (int32_t)bm->free_q.size();
}

PKV_API int32_t pkv_bm_ref_counts(const pkv_block_manager *bm, int32_t *counts, int32_t cap) {
    if (!bm || (cap > 0 && !counts)) return PKV_ERR_NULL;
    for (int32_t b = 0; b < cap && b < bm->num_blocks; ++b) counts[b] = bm->ref[b];
    return bm->num_blocks;
}

PKV_API int pkv_bm_get_stats(const pkv_block_manager *bm, pkv_bm_stats *out) {
    if (!bm || !out) return PKV_ERR_NULL;
    return guarded([&] {
        // live slots: each (block, slot) pair counted once, shared or not
        std::vector<uint8_t> live((size_t)bm->num_blocks * bm->block_size, 0);
        int64_t n = 0;
        for (const auto &kv : bm->seqs) {
            const auto &s = kv.second;
            for (int64_t t = 0; t < s.len; ++t) {
                const int64_t p = s.offset + t;
                const size_t idx = (size_t)s.blocks[p / bm->block_size] * bm->block_size + p % bm->block_size;
                if (!live[idx]) {
                    live[idx] = 1;
                    ++n;
                }
            }
        }
        out->num_blocks = bm->num_blocks;
        out->block_size = bm->block_size;
        out->free_blocks = bm->free_q.size();
        out->used_blocks = bm->used();
        out->peak_used_blocks = bm->peak_used;
        out->live_tokens = n;
        out->num_seqs = (int64_t)bm->seqs.size();
        return PKV_OK;
    });
}

}  // extern "C"
