// kernels_decode.hip -- fused paged decode attention for gfx950.
//
// Computes, for every sequence s and query head h (kv head g = h / G):
//   out[s,h,:] = softmax_t(scale * q[s,h,:] . K_t[g,:]) . V_t[g,:]
// reading K_t and V_t in place from the paged pool through the block table
// (the fused kernel of [P1 "comparison with vLLM"] and [P3 sec. 3.1], whose
// result is gather-then-attention [P2 sec. 2.3]).
//
// Sources:
//   [P1] mini-vllm tutorial, "step14_2 - index_select gather"
//   [P2] "vLLM PagedAttention source notes"
//   [P3] mini-runtime, chapter 12 "Paged KV Cache"
//
// Work decomposition
//   Splits are ranges of flat table positions: split j of a sequence covers
//   positions [j*S, (j+1)*S) intersected with [offset, offset + seq_len)
//   (logical token t sits at flat position offset + t).  A work item is
//   (sequence, kv head, split); one wavefront owns it and all G query heads
//   of that kv head, so every K/V row is read from HBM once and used G
//   times.  A workgroup holds up to 4 wavefronts = a group of kv heads of
//   one (sequence, split): they share the block-table entries, staged in
//   LDS once per workgroup, and read each block's layer slice together.
//   Two schedules map workgroups to work items:
//   - split: one workgroup per (sequence, split, head group), split S chosen
//     by the host from max_seq_len; workgroups are renumbered so that the
//     splits of one sequence land on different XCDs;
//   - device-planned split (plan_item below): every workgroup reads all
//     lengths, picks S so the pieces fit two workgroups per compute unit,
//     and takes one piece.
//
// bf16 kernel, per 16-position chunk of one block:
//   QK:  S^T = K_chunk (16 x D) . Q^T (D x 16 heads, G real) with
//        v_mfma_f32_16x16x32_bf16.  Lane l loads K row l%16, elements
//        32j + 8*(l/16) .. +8 for step j -- exactly the MFMA operand layout,
//        so K goes from HBM to the matrix core with no shuffling.  Lane l
//        then holds the scores of tokens 4*(l/16) .. +3 for head l%16.
//   softmax: scores live in the exp2 domain (scale*log2 e folded in).  Each
//        head keeps a reference max m that only moves when a chunk's max
//        exceeds it by more than 8 (so p <= 256; the result is exact
//        whatever the reference, since acc and l share it); the P.V
//        accumulators are rescaled only on such a move (a wave-uniform
//        branch, rare after the first chunks).  The chunk max across the
//        four 16-lane rows uses the gfx950 row swaps.
//   PV:  V goes HBM -> LDS directly (global_load_lds, 16 bytes per lane) in
//        a padded tile; the transposing LDS read gives the B operand and
//        O (16 heads x D) += P . V runs as v_mfma_f32_16x16x16_bf16, with P
//        (the score layout is the A-operand layout) rounded to bf16.
//   Loads are unconditional and in bounds: a missing block reads block 0 and
//   prefetches past the end re-read the last chunk.  Masked positions
//   (before the offset, past seq_len, invalid table entry) get score -inf
//   and their V tile rows are zeroed, so poisoned (NaN) pool slots cannot
//   leak in.  A ring of chunks keeps the next ones' loads in flight while
//   one is computed.
//
// int8 kernel (decode_q8_kernel): QK^T on the int8 matrix cores over the
// codes as loaded, V codes converted to bf16 into the same tile layout; see
// its section below.
//
// fp32 kernel (VALU): row layout for K and V, dot products reduced over the
//   lanes of a row with DPP, per-chunk wave-uniform max; used for the fp32
//   pool dtype.
//
// Split-K: with more than one split per sequence, each work item writes its
// unnormalised (m, l, acc) to the workspace, and the splits of each
// (sequence, query head) are merged in split order:
//   M = max_j m_j,  L = sum_j l_j 2^(m_j - M),  O = sum_j acc_j 2^(m_j - M) / L
// by the work item that finishes last (at most 16 splits) or by a second
// kernel (reduce_kernel).  With one split the work item normalises and
// writes the output itself.  The MFMA kernels at head_dim 128 keep the acc
// rows for the in-kernel merge in half precision, each row re-referenced by
// a power of two (see "Split records in half precision").
#include "attn_common.h"

namespace pkv {


// (sequence, split, head group) of this workgroup.  Logical order: split
// slowest, then head group, then sequence, so the splits that exist only
// for long sequences (most of them empty) are dispatched last.  Workgroups
// are dealt round-robin to the 8 XCDs (XCD = blockIdx % 8); within each
// aligned group of 8 logical items the XCD is rotated by the group's
// (split, head group) index, so the splits of one sequence land on
// different XCDs and every XCD gets a like share of the live work.
struct Item {
    int seq, split, hg;
};

__device__ __forceinline__ Item work_item(const DecodeArgs &a) {
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int row = bid & ~7;
    int lid = bid;
    if (row + 8 <= nwg) lid = row | ((bid - row / a.num_seqs) & 7);
    Item it;
    it.seq = lid % a.num_seqs;
    const int rest = lid / a.num_seqs;
    it.hg = rest % a.head_groups;
    it.split = rest / a.head_groups;
    return it;
}

// Flat-position range [lo, hi) of split j: [j*S, (j+1)*S) n [off, off+L).
// `whole` is false when the caller's length or offset broke the contract
// (length above max_seq_len, offset outside [0, block_size)) and was clamped.
struct Range {
    int64_t lo, hi, off, len;
    bool whole;
};

// A sequence's length clamped to [0, max_seq_len] and its offset to
// [0, block_size): the grid and the workspace are sized from max_seq_len,
// so every split index and merge count stays inside them whatever the
// device-resident values hold.
__device__ __forceinline__ void clamp_len_off(const DecodeArgs &a, int64_t &L, int64_t &off, bool &whole) {
    const int64_t bsm = (1ll << a.pool.lbs) - 1;
    const int64_t L0 = L, o0 = off;
    L = L < 0 ? 0 : (L > a.max_len ? (int64_t)a.max_len : L);
    off = off < 0 ? 0 : (off > bsm ? bsm : off);
    whole = L == L0 && off == o0;
}

__device__ __forceinline__ Range split_range(const DecodeArgs &a, int seq, int split) {
    Range R;
    int64_t L = a.seq_lens[seq];
    int64_t off = a.offsets[seq];
    clamp_len_off(a, L, off, R.whole);
    R.len = L;
    R.off = off;
    const int64_t S = a.split_tokens;
    R.lo = max((int64_t)split * S, R.off);
    R.hi = min((int64_t)(split + 1) * S, R.off + L);
    return R;
}

// Stage the table entries that cover [lo, hi) into bt_s (entry jb0 first);
// ids outside the pool or past the table become -1.  All threads of the
// workgroup call this.
__device__ __forceinline__ int64_t stage_table(const DecodeArgs &a, int seq, const Range &R,
                                               int32_t *bt_s) {
    const int lbs = a.pool.lbs;
    const int64_t jb0 = R.lo >> lbs;
    const int nbt = R.hi > R.lo ? (int)(((R.hi - 1) >> lbs) - jb0 + 1) : 0;
    for (int i = threadIdx.x; i < nbt; i += blockDim.x) {
        const int64_t j = jb0 + i;
        int32_t b = -1;
        if (j >= 0 && j < a.bt_stride) {
            b = a.block_tables[(int64_t)seq * a.bt_stride + j];
            if (b < 0 || b >= a.pool.num_blocks) b = -1;
        }
        bt_s[i] = b;
    }
    __syncthreads();
    return jb0;
}


template <int DT>
__device__ __forceinline__ void store_out(char *dst, const float *v, int n);
template <>
__device__ __forceinline__ void store_out<0>(char *dst, const float *v, int n) {
    if (n == 2)
        *reinterpret_cast<float2 *>(dst) = make_float2(v[0], v[1]);
    else
        *reinterpret_cast<float *>(dst) = v[0];
}
template <>
__device__ __forceinline__ void store_out<1>(char *dst, const float *v, int n) {
    if (n == 2)
        *reinterpret_cast<uint32_t *>(dst) = f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16);
    else
        *reinterpret_cast<uint16_t *>(dst) = (uint16_t)f32_to_bf16_bits(v[0]);
}


// Split partials are shared between workgroups that may run on different
// XCDs, each with its own L2.  They are written and read with device-scope
// accesses (stores write through, loads bypass the non-coherent caches), so
// no cache writeback or invalidation is needed around the hand-over.
__device__ __forceinline__ void st_dev(float *p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev2(float *p, float x, float y) {
    const uint64_t u = (uint64_t)__float_as_uint(x) | ((uint64_t)__float_as_uint(y) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t *>(p), u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float *p) {
    return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 ld_dev2(const float *p) {
    const uint64_t u = __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<float *>(p)),
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)u), __uint_as_float((uint32_t)(u >> 32)));
}
__device__ __forceinline__ uint64_t ld_dev_u64(const void *p) {
    return __hip_atomic_load(reinterpret_cast<uint64_t *>(const_cast<void *>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Split records in half precision (the MFMA kernels at head_dim 128).
//
// A record is (m, l, acc) per query head: the reference max, the
// denominator and the unnormalised accumulator row.  For any integer k,
// (m + k, l * 2^-k, acc * 2^-k) merges exactly like (m, l, acc), since the
// merge weighs a record's acc and l by the same 2^(m - M).  Each head row
// takes k from its largest finite magnitude, which puts that element in
// [2^14, 2^15): the row then fits half precision, and every element is
// stored to within 2^-12 of the row's largest (round to nearest even).  k
// is clamped to [-100, 110], so l * 2^-k stays a normal float (l lies in
// [1, 2^24]).  Infinities and NaNs are carried through.  The rows then move
// half the bytes of single precision through the split hand-over, whose
// stores and loads are what the in-kernel merge waits on.
// ---------------------------------------------------------------------------
// Which records use them: those of the MFMA kernels (bf16, int8 and int4
// pools) at head_dim 128 that the in-kernel merge reads (at most 16 splits
// per sequence).  With the writer and merge below, the 32 x U[128, 2048]
// token batch, where the in-kernel merge runs, went from 38.8 to 36.1 us
// (bf16) and from 28.5 to 25.4 us (int8) against single-precision records.
// Records for reduce_kernel stay in single precision: half precision there
// measured slower on 8 x 32768 tokens (bf16 175.8 -> 178.6 us, int8 101.0
// -> 104.1 us, same process).
template <int D>
constexpr bool kRecordsHalf = D == 128;

typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t f16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), f16x2));
}
__device__ __forceinline__ f32x2 f16x2_to_f32(uint32_t u) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, u), f32x2);
}
__device__ __forceinline__ float finite_abs(float x) {
    const float a = fabsf(x);
    return a != __builtin_huge_valf() ? a : 0.0f;
}
// max over the 16 lanes of a row (NaN-ignoring)
__device__ __forceinline__ float row_max16(float x) {
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return x;
}
// exponent shift k of a row whose largest finite magnitude is amax
__device__ __forceinline__ int rec_shift(float amax) {
    const int e = __builtin_amdgcn_frexp_expf(amax);  // amax = f 2^e, f in [0.5, 1); 0 for 0
    return min(max(e - 15, -100), 110);
}

// A sequence with no tokens attends to nothing: its output rows are zero.
// Written by the split-0 workgroup of each head group (multi-split case).
template <int DT, int D, int G>
__device__ void zero_outputs(const DecodeArgs &a, int seq, int hg) {
    constexpr int E = Elem<DT>::kBytes;
    const int64_t n = (int64_t)a.heads_per_wg * G * D * E / 4;
    uint32_t *o = reinterpret_cast<uint32_t *>(
        a.out + ((int64_t)seq * a.num_q_heads + (int64_t)hg * a.heads_per_wg * G) * D * E);
    for (int64_t i = threadIdx.x; i < n; i += blockDim.x) o[i] = 0u;
}

// ---------------------------------------------------------------------------
// Device-planned split schedule (bf16 and int8 pools, a.plan = number of
// workgroups).  The
// host knows only the largest sequence length, so a split it picks cannot
// fit the batch: with the lengths of the decode batch the automatic
// 256-token split leaves 30 of 256 compute units without a live work item
// while 96 hold two, most of them full.  Here every workgroup reads all
// lengths and offsets (the memory round trip it already makes for its
// own), picks the smallest split S (a multiple of 16, at least
// a.split_tokens) whose pieces -- the splits of "Work decomposition"
// above, per (sequence, head group) -- fit the grid, and takes piece number
// blockIdx.x in an order that spreads them: pieces of exactly S positions
// from the front of the grid, shorter ones (a sequence's first and last)
// from the back.  With two resident workgroups per compute unit,
// workgroups b and b + gridDim/2 share one, so a compute unit holds at most
// two pieces of at most S positions each.
// The host guarantees a feasible S: gridDim.x >= n * head_groups *
// a.max_splits (then S = a.split_tokens fits), or gridDim.x >= 4 * n *
// head_groups (then the bound below fits), n <= kPlanMaxSeqs (one per lane
// of one wavefront) and positions below 2^24.
// The whole plan runs in wavefront 0, in registers: this is the latency
// before the first table entry can be fetched.
// ---------------------------------------------------------------------------

// floor(x / d) for 0 <= x < 2^24, 16 <= d or x / d < 2^20, d > 0, from an
// approximate reciprocal (relative error below 2^-22, so the float
// quotient is within 1 of the true one) and one correction step.
__device__ __forceinline__ int32_t udiv24(int32_t x, int32_t d, float rcp) {
    int32_t q = (int32_t)((float)x * rcp);
    const int32_t r = x - q * d;
    if (r < 0) --q;
    else if (r >= d) ++q;
    return q;
}

// Pieces of one sequence (offset o, length L) at split S: first and last
// split index, the first full piece and the number of full pieces (a piece
// is full when it covers all S positions of its split), and the number of
// the others (0, 1 or 2: the first and the last piece).
struct SeqPieces {
    int32_t j0, j1, jf0, nf, nq;
};

__device__ __forceinline__ SeqPieces seq_pieces(int32_t L, int32_t o, int32_t S, float rcp) {
    SeqPieces p{0, -1, 0, 0, 0};
    if (L <= 0) return p;
    p.j0 = udiv24(o, S, rcp);
    p.j1 = udiv24(o + L - 1, S, rcp);
    const bool f0 = p.j0 * S >= o && (p.j0 + 1) * S <= o + L;
    const bool f1 = p.j1 * S >= o && (p.j1 + 1) * S <= o + L;
    p.jf0 = f0 ? p.j0 : p.j0 + 1;
    const int32_t jf1 = f1 ? p.j1 : p.j1 - 1;
    p.nf = jf1 >= p.jf0 ? jf1 - p.jf0 + 1 : 0;
    p.nq = (p.j1 - p.j0 + 1) - p.nf;
    return p;
}

// Row shift-right by K within rows of 16 lanes; lanes with no source read 0.
template <int K>
__device__ __forceinline__ int32_t row_shr(int32_t v) {
    return __builtin_amdgcn_update_dpp(0, v, 0x110 + K, 0xf, 0xf, true);
}

// Inclusive prefix sum over the 64 lanes of a wavefront (DPP within rows
// of 16, then the row totals from lanes 15, 31 and 47).
__device__ __forceinline__ int32_t wave_incl_scan(int32_t v) {
    v += row_shr<1>(v);
    v += row_shr<2>(v);
    v += row_shr<4>(v);
    v += row_shr<8>(v);
    const int row = (threadIdx.x & 63) >> 4;
    const int32_t r0 = __builtin_amdgcn_readlane(v, 15);
    const int32_t r1 = __builtin_amdgcn_readlane(v, 31);
    const int32_t r2 = __builtin_amdgcn_readlane(v, 47);
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

__device__ __forceinline__ int32_t wave_total(int32_t v) {
    return __builtin_amdgcn_readlane(wave_incl_scan(v), 63);
}

struct PlanOut {
    int32_t seq, g, j, len, off, S, have, whole;
};

// Sets it, R and S of this workgroup; false if it has no piece.  Uses
// scratch (the table staging buffer, at least kPlanMaxSeqs entries) for
// the clamped lengths and ends with a barrier, after which scratch may be
// reused.  Empty sequences' outputs are zeroed here (sequence s by
// workgroup s % gridDim.x).  All threads of the workgroup call this.
// Lane t of wavefront 0 holds sequence t (n <= 64).
template <int D, int G>
__device__ bool plan_item(const DecodeArgs &a, int32_t *scratch, Item &it, Range &R, int64_t &S_out) {
    static_assert(kPlanMaxSeqs <= 64, "one sequence per lane");
    __shared__ PlanOut po;
    const int n = a.num_seqs;
    const int nwg = gridDim.x;
    if (threadIdx.x < 64) {
        const int lane = threadIdx.x;
        const int HG = a.head_groups;
        const int32_t bsm = (1 << a.pool.lbs) - 1;
        const bool live = lane < n;
        int32_t L = live ? a.seq_lens[lane] : 0;
        int32_t O = live ? a.offsets[lane] : 0;
        const int32_t L0 = L, O0 = O;
        L = L < 0 ? 0 : (L > a.max_len ? a.max_len : L);
        O = O < 0 ? 0 : (O > bsm ? bsm : O);
        const int32_t whole = L == L0 && O == O0;
        if (live) scratch[lane] = L;
        // total length: below 64 * 2^24 < 2^31 (the float value's rounding is
        // within the bounds' margins)
        const float totf = (float)wave_total(L);
        // pieces of all pairs at split S
        auto count = [&](int32_t S) -> int32_t {
            const float rcp = __builtin_amdgcn_rcpf((float)S);
            const int32_t c = L > 0 ? udiv24(O + L - 1, S, rcp) - udiv24(O, S, rcp) + 1 : 0;
            return wave_total(c) * HG;
        };
        const int32_t smin = a.split_tokens;
        // lower end: the pieces number at least HG * total / S, so S >=
        // HG * total / nwg (a float estimate; one 16-step below is safe)
        int32_t lo = (int32_t)((float)HG * totf / (float)nwg) - 16;
        lo = lo < smin ? smin : lo;
        lo = (lo + 15) >> 4;
        // upper end, feasible: S = smin when the grid holds every pair's
        // a.max_splits pieces; else pieces <= HG * (total / S + 2 n) <= nwg
        // for S >= HG * total / (nwg - 2 HG n), rounded up with margin
        int32_t hi;
        if (nwg >= n * HG * a.max_splits) {
            hi = smin >> 4;
        } else {
            const float room = (float)(nwg - 2 * HG * n);  // >= 2 HG n (host)
            hi = (int32_t)((float)HG * totf / room * 1.0001f) + 2;
            hi = (hi + 15) >> 4;
            hi = hi < (smin >> 4) ? (smin >> 4) : hi;
        }
        if (lo > hi) lo = hi;
        if (count(lo * 16) > nwg) {
            ++lo;
            while (lo < hi) {
                const int32_t mid = (lo + hi) >> 1;
                if (count(mid * 16) <= nwg) hi = mid;
                else lo = mid + 1;
            }
        }
        const int32_t S = lo * 16;
        const SeqPieces P = seq_pieces(L, O, S, __builtin_amdgcn_rcpf((float)S));
        // running totals of full (sf) and other (sq) pieces
        const int32_t sf = wave_incl_scan(P.nf), sq = wave_incl_scan(P.nq);
        const int32_t Fs = __builtin_amdgcn_readlane(sf, 63), Qs = __builtin_amdgcn_readlane(sq, 63);
        const int32_t b = blockIdx.x;
        PlanOut r{0, 0, 0, 0, 0, S, 0, 1};
        const bool full = b < HG * Fs;
        if (full || b >= nwg - HG * Qs) {
            const int32_t tot_p = full ? Fs : Qs;
            const int32_t x = full ? b : nwg - 1 - b;
            const int32_t g = udiv24(x, tot_p, __builtin_amdgcn_rcpf((float)tot_p));
            const int32_t k = x - g * tot_p;  // rank among this head group's pieces
            const int32_t incl = full ? sf : sq;
            const int32_t cnt = full ? P.nf : P.nq;
            const uint64_t hit = __ballot(cnt > 0 && incl - cnt <= k && k < incl);
            const int ln = __builtin_ctzll(hit);  // exactly one lane
            const int32_t base = __builtin_amdgcn_readlane(incl - cnt, ln);
            const int32_t j0 = __builtin_amdgcn_readlane(P.j0, ln);
            const int32_t j1 = __builtin_amdgcn_readlane(P.j1, ln);
            const int32_t jf0 = __builtin_amdgcn_readlane(P.jf0, ln);
            const int32_t nf = __builtin_amdgcn_readlane(P.nf, ln);
            r.seq = ln;
            r.g = g;
            // the others, in order: the first piece unless it is full, then the last
            r.j = full ? jf0 + (k - base) : ((k == base && !(nf > 0 && jf0 == j0)) ? j0 : j1);
            r.len = __builtin_amdgcn_readlane(L, ln);
            r.off = __builtin_amdgcn_readlane(O, ln);
            r.whole = __builtin_amdgcn_readlane(whole, ln);
            r.have = 1;
        }
        if (lane == 0) po = r;
    }
    __syncthreads();
    const PlanOut r = po;
    // outputs of empty sequences
    for (int t = blockIdx.x; t < n; t += nwg)
        if (scratch[t] == 0)
            for (int g = 0; g < a.head_groups; ++g) zero_outputs<1, D, G>(a, t, g);
    if (r.have) {
        it.seq = r.seq;
        it.hg = r.g;
        it.split = r.j;
        R.len = r.len;
        R.off = r.off;
        R.whole = r.whole != 0;
        R.lo = max((int64_t)r.j * r.S, R.off);
        R.hi = min((int64_t)(r.j + 1) * r.S, R.off + R.len);
    }
    S_out = r.S;
    __syncthreads();
    return r.have != 0;
}

// Merge of partial results into out for the G query heads of one kv head:
//   M = max_i m_i,  w_i = 2^(m_i - M),
//   out = (sum_i w_i acc_i) / (sum_i w_i l_i)
// over n records.  Record i of query head g has its (m, l) at
// ml + (slot(i) * hstride + g) * 2 and its acc row at
// acc + (slot(i) * hstride + g) * D.  One wavefront; lane covers D/64
// consecutive output elements.  Records are summed in index order, so the
// result does not depend on which workgroup runs the merge.  Up to 64
// records, the (m, l) pairs (lane i: record i) and the first RB records'
// acc rows are loaded together, so the merge costs one memory round trip
// per RB records.  (This single-precision merge serves head_dim 64 and the
// fp32 pools; at head_dim 128 the MFMA kernels use merge_records_h.  When
// it served the decode batch, 13 records, per-workgroup timestamps put it
// at 3.6 us from the count to its stores, about 2.5 us of that the wait for
// the device-scope loads; the cross-lane max and sum as DPP + row swaps,
// and staged records read four at a time, had taken it from 4.3 us.)
template <int DT, int D, int G, typename Slot>
__device__ void merge_records(char *out_row0, const float *ml, const float *accb, int64_t hstride,
                              int n, Slot slot, char *lds = nullptr, int lds_bytes = 0) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int PL = D / 64;
    // acc records per batch: 64 values per lane, so the merge needs no more
    // registers than the attention loop (occupancy stays at 2 waves/SIMD)
    constexpr int RB = (64 / (G * PL)) < 16 ? (64 / (G * PL) > 0 ? 64 / (G * PL) : 1) : 16;
    static_assert(PL == 1 || PL == 2, "head_dim");
    // the G acc rows of one record are contiguous (G * D floats)
    constexpr int RECB = G * D * 4;
    // staged only when a record is whole 1 KiB tile-load instructions
    constexpr bool kStage = RECB % 1024 == 0;
    const int lane = threadIdx.x & 63;
    const float *acc = accb + lane * PL;
    // Records RB .. RB + LR - 1 go global -> LDS (the wavefront's own free
    // LDS, lds_bytes of it) in the same memory round trip as the first RB,
    // with the same device-scope (sc1) loads; past that, batches of RB.
    const int LR = kStage && n <= 64 ? min(lds_bytes / RECB, max(n - RB, 0)) : 0;

    float M[G], w[G], den[G], o[G][PL];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        M[g] = kNegInf;
        den[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < PL; ++e) o[g][e] = 0.0f;
    }
    // acc rows of records b .. b+RB-1 (none past the last record)
    auto load_batch = [&](int b, float (&x)[RB][G][PL]) {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
            const float *src = acc + slot(min(b + k, n - 1)) * hstride * D;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (b + k >= n) {
#pragma unroll
                    for (int e = 0; e < PL; ++e) x[k][g][e] = 0.0f;
                } else if constexpr (PL == 2) {
                    const float2 t = ld_dev2(src + g * D);
                    x[k][g][0] = t.x;
                    x[k][g][1] = t.y;
                } else {
                    x[k][g][0] = ld_dev(src + g * D);
                }
            }
        }
    };
    auto add_batch = [&](int b, const float (&x)[RB][G][PL], const float (&wl)[G]) {
#pragma unroll
        for (int k = 0; k < RB; ++k) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                // weight of record b + k: lane (b + k) % 64 holds it
                const float wk = b + k < n ? lane_value(wl[g], (b + k) & 63) : 0.0f;
#pragma unroll
                for (int e = 0; e < PL; ++e) o[g][e] = fmaf(wk != 0.0f ? x[k][g][e] : 0.0f, wk, o[g][e]);
            }
        }
    };

    if (n <= 64) {
        for (int r = 0; r < LR; ++r) {
            const char *src = reinterpret_cast<const char *>(accb + slot(RB + r) * hstride * D);
#pragma unroll
            for (int i = 0; i < (kStage ? RECB / 1024 : 0); ++i)
                __builtin_amdgcn_global_load_lds(const_cast<char *>(src) + 1024 * i + 16 * lane,
                                                 (__attribute__((address_space(3))) void *)(lds + r * RECB + 1024 * i),
                                                 16, 0, 16 /* sc1 */);
        }
        float mv[G], lv[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            mv[g] = kNegInf;
            lv[g] = 0.0f;
        }
        if (lane < n) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float2 v = ld_dev2(ml + (slot(lane) * hstride + g) * 2);
                mv[g] = v.x;
                lv[g] = v.y;
            }
        }
        float x[RB][G][PL];
        load_batch(0, x);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            M[g] = wave_max(mv[g]);
            w[g] = mv[g] != kNegInf ? fast_exp2(mv[g] - M[g]) : 0.0f;
            den[g] = lane < n ? lv[g] * w[g] : 0.0f;
        }
        add_batch(0, x, w);
        if (LR > 0) {
            // the copy engine's writes are not tracked by the compiler
            __builtin_amdgcn_s_waitcnt((0x7 << 4) | (0xF << 8));
            wave_lds_order();
            // four records per step, so their LDS reads are in flight together
            for (int r0 = 0; r0 < LR; r0 += 4) {
                float y[4][G][PL];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float *row =
                            reinterpret_cast<const float *>(lds + min(r0 + k, LR - 1) * RECB) + g * D + lane * PL;
#pragma unroll
                        for (int e = 0; e < PL; ++e) y[k][g][e] = row[e];
                    }
                }
#pragma unroll
                for (int k = 0; k < 4; ++k) {
#pragma unroll
                    for (int g = 0; g < G; ++g) {
                        const float wk = r0 + k < LR ? lane_value(w[g], (RB + r0 + k) & 63) : 0.0f;
#pragma unroll
                        for (int e = 0; e < PL; ++e) o[g][e] = fmaf(wk != 0.0f ? y[k][g][e] : 0.0f, wk, o[g][e]);
                    }
                }
            }
            wave_lds_order();
        }
        for (int b = RB + LR; b < n; b += RB) {
            load_batch(b, x);
            add_batch(b, x, w);
        }
    } else {
        for (int i = lane; i < n; i += 64) {
            const int64_t r = slot(i) * hstride;
#pragma unroll
            for (int g = 0; g < G; ++g) M[g] = fmaxf(M[g], ld_dev(ml + (r + g) * 2));
        }
#pragma unroll
        for (int g = 0; g < G; ++g) M[g] = wave_max(M[g]);
        for (int ic = 0; ic < n; ic += 64) {
            const int i = ic + lane;
#pragma unroll
            for (int g = 0; g < G; ++g) {
                w[g] = 0.0f;
                if (i < n) {
                    const float2 v = ld_dev2(ml + (slot(i) * hstride + g) * 2);
                    if (v.x != kNegInf) w[g] = fast_exp2(v.x - M[g]);
                    den[g] = fmaf(v.y, w[g], den[g]);
                }
            }
            const int nu = min(64, n - ic);
            float x[RB][G][PL];
            for (int b = 0; b < nu; b += RB) {
                load_batch(ic + b, x);
                add_batch(ic + b, x, w);
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float L = wave_sum(den[g]);
        float v[PL];
#pragma unroll
        for (int e = 0; e < PL; ++e) v[e] = L > 0.0f ? o[g][e] / L : 0.0f;
        store_out<DT>(out_row0 + ((int64_t)g * D + lane * PL) * E, v, PL);
    }
}

// merge_records for half-precision records (head_dim 128) of the in-kernel
// merge: n <= kFusedMergeMaxSplits records, record i's row of query head g
// at rec0 + (i * hstride + g) * D halves, its (m, l) at ml + (i * hstride +
// g) * 2.  An 8-byte load covers two 256-byte rows: lane (hh, c) holds
// columns 4c .. 4c+3 of head 2q + hh of each head pair q.  The
// kFusedMergeMaxSplits slots are unrolled in groups of 4; a group past the
// n records is skipped whole.  Slot k reads record min(k, n - 1) (a scalar
// offset), and slots past n weigh 0, their words zeroed like any
// zero-weight record's (as merge_records does).  The (m, l) pairs (lane i:
// record i) and all rows are loaded together: at G <= 4 the merge is one
// memory round trip.  Summed in record order, like merge_records.
constexpr int kMergeGroup = 4;

template <int DT, int D, int G>
__device__ void merge_records_h(char *out_row0, const float *ml, const uint16_t *rec0, int64_t hstride, int n) {
    static_assert(D == 128, "half-precision records: head_dim 128");
    constexpr int E = Elem<DT>::kBytes;
    constexpr int HP = (G + 1) / 2;  // head pairs
    constexpr int NS = kFusedMergeMaxSplits;
    constexpr int kSC1 = 16;  // cache-policy bit sc1 of a buffer access (device scope, as ld_dev)
    const int lane = threadIdx.x & 63;
    const int hh = lane >> 5;
    const int c0 = 4 * (lane & 31);

    float mv[G], lv[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        mv[g] = kNegInf;
        lv[g] = 0.0f;
    }
    if (lane < n) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const float2 v = ld_dev2(ml + ((int64_t)lane * hstride + g) * 2);
            mv[g] = v.x;
            lv[g] = v.y;
        }
    }
    // (readfirstlane returns a signed int: each half of the address is
    // widened through uint32_t.)
    const uint64_t u = reinterpret_cast<uint64_t>(rec0);
    const uint32_t ulo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t uhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    const uint32_t stride = (uint32_t)hstride * D * 2;  // bytes between records
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(((uint64_t)uhi << 32) | ulo), 0, (int)(n * stride), 0x00020000);
    // lanes of a missing second head (odd G) read head G - 1 and are not stored
    uint32_t voff[HP];
#pragma unroll
    for (int q = 0; q < HP; ++q) voff[q] = (uint32_t)(min(2 * q + hh, G - 1) * D + c0) * 2;
    // slots in groups of kMergeGroup: a group past the n records is neither
    // loaded nor summed (one wave-uniform test on n per group)
    const int nu = __builtin_amdgcn_readfirstlane(n);
    u32x2v x[NS][HP];
#pragma unroll
    for (int k0 = 0; k0 < NS; k0 += kMergeGroup) {
        if (k0 >= nu) break;
#pragma unroll
        for (int k = k0; k < k0 + kMergeGroup; ++k) {
            const uint32_t rk = (uint32_t)min(k, nu - 1) * stride;
#pragma unroll
            for (int q = 0; q < HP; ++q)
                x[k][q] = __builtin_bit_cast(u32x2v,
                                             __builtin_amdgcn_raw_buffer_load_b64(rs, voff[q] + rk, 0, kSC1));
        }
    }
    float w[G], den[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float M = wave_max(mv[g]);
        w[g] = mv[g] != kNegInf ? fast_exp2(mv[g] - M) : 0.0f;
        den[g] = lane < n ? lv[g] * w[g] : 0.0f;
    }
    float o[HP][4];
#pragma unroll
    for (int q = 0; q < HP; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[q][e] = 0.0f;
#pragma unroll
    for (int k = 0; k < NS; ++k) {
        if (k % kMergeGroup == 0 && k >= nu) break;
#pragma unroll
        for (int q = 0; q < HP; ++q) {
            // weight of record k for this lane's head (lane k holds it; 0 past
            // the n records)
            const float wa = lane_value(w[2 * q], k);
            const float wb = 2 * q + 1 < G ? lane_value(w[2 * q + 1 < G ? 2 * q + 1 : 0], k) : 0.0f;
            const float wk = hh ? wb : wa;
            const bool use = wk != 0.0f;
            // each half widened inside the fma (v_fma_mix_f32)
            const f16x2 lo = __builtin_bit_cast(f16x2, use ? x[k][q][0] : 0u);
            const f16x2 hi = __builtin_bit_cast(f16x2, use ? x[k][q][1] : 0u);
            o[q][0] = fmaf((float)lo[0], wk, o[q][0]);
            o[q][1] = fmaf((float)lo[1], wk, o[q][1]);
            o[q][2] = fmaf((float)hi[0], wk, o[q][2]);
            o[q][3] = fmaf((float)hi[1], wk, o[q][3]);
        }
    }
#pragma unroll
    for (int q = 0; q < HP; ++q) {
        // both denominators as scalars (a select between two elements of an
        // array became an indexed stack access)
        const float La = wave_sum(den[2 * q]);
        const float Lb = 2 * q + 1 < G ? wave_sum(den[2 * q + 1 < G ? 2 * q + 1 : 0]) : 0.0f;
        const int g = 2 * q + hh;
        if (g >= G) continue;
        const float Lg = hh ? Lb : La;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = Lg > 0.0f ? o[q][e] / Lg : 0.0f;
        char *dst = out_row0 + ((int64_t)g * D + c0) * E;
        if constexpr (DT == 1) {
            *reinterpret_cast<u32x2v *>(dst) = u32x2v{f32_to_bf16_bits(v[0]) | (f32_to_bf16_bits(v[1]) << 16),
                                                      f32_to_bf16_bits(v[2]) | (f32_to_bf16_bits(v[3]) << 16)};
        } else {
            *reinterpret_cast<f32x4 *>(dst) = f32x4{v[0], v[1], v[2], v[3]};
        }
    }
}

// Count one finished contribution to a merge group; true, in every thread,
// for the workgroup that completes the count of `expected`.  Partials are
// written with device-scope stores and each wavefront waits until its
// stores are complete before the barrier, so they are visible device-wide
// before the count is published.  The completing workgroup puts the counter
// back to zero for the next call.  Called by all threads of the workgroup.
//
// Why relaxed: every access to the shared partials is itself an
// agent-scope atomic (stores write through to the device-coherent level,
// loads bypass the XCD's non-coherent L2), the s_waitcnt below holds each
// wavefront until its stores have completed there, and the completing
// workgroup issues its loads only after the count has returned (barrier in
// between).  So the hand-over needs no cache maintenance.  An agent-scope
// release on the count (with an acquire fence in the completing workgroup)
// would add an L2 writeback to every contribution: measured on MI355X,
// same process, decode batch 37.5 -> 52.3 us, prefix sharing 88.5 ->
// 107.1 us, int8 decode batch 28.8 -> 44.6 us.
__device__ bool count_in(uint32_t *cnt, uint32_t expected) {
    __shared__ int last_s;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t done = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = done + 1 == expected;
        if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        last_s = last;
    }
    __syncthreads();
    return last_s != 0;
}

// End of a multi-split work item (split schedule): count the split in for
// (sequence, head group); the workgroup that completes the count merges the
// live splits j0 .. j1 of the sequence, each wavefront the G query heads of
// its kv head.
// H: the records are in half precision (see "Split records in half
// precision").
template <int DT, int D, int G, bool H = false>
__device__ void finish_split(const DecodeArgs &a, const Item &it, const Range &R, int64_t S,
                             char *lds = nullptr, int lds_bytes = 0) {
    constexpr int E = Elem<DT>::kBytes;
    const int j0 = (int)(R.off / S);
    const int j1 = (int)((R.off + R.len - 1) / S);
    if (!count_in(a.ws_cnt + (int64_t)it.seq * a.head_groups + it.hg, (uint32_t)(j1 - j0 + 1))) return;
    const int h = it.hg * a.heads_per_wg + (threadIdx.x >> 6);
    const int64_t hq0 = (int64_t)h * G;
    const int64_t item0 = (int64_t)it.seq * a.max_splits * a.num_q_heads + hq0;
    char *out0 = a.out + ((int64_t)it.seq * a.num_q_heads + hq0) * D * E;
    if constexpr (H) {
        const int64_t r0 = item0 + (int64_t)j0 * a.num_q_heads;  // record j0
        merge_records_h<DT, D, G>(out0, a.ws_ml + r0 * 2, reinterpret_cast<const uint16_t *>(a.ws_acc) + r0 * D,
                                  a.num_q_heads, j1 - j0 + 1);
    } else {
        merge_records<DT, D, G>(out0, a.ws_ml + item0 * 2, a.ws_acc + item0 * D, a.num_q_heads, j1 - j0 + 1,
                                [=](int i) { return (int64_t)(j0 + i); }, lds, lds_bytes);
    }
}

// ---------------------------------------------------------------------------
// fp32 pools: VALU kernel.
// ---------------------------------------------------------------------------
template <int DT, int D, int G>
__global__ __launch_bounds__(256) void decode_valu_kernel(DecodeArgs a) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int VEC = 16 / E;               // elements per 16-byte piece
    constexpr int LPR = D / VEC;              // lanes per kv-head row
    constexpr int RPI = 64 / LPR;             // rows per wavefront pass
    constexpr int NP = kChunkTokens / RPI;    // passes per chunk
    static_assert(LPR >= 4 && LPR <= 64 && RPI <= kChunkTokens, "head_dim out of range");

    __shared__ int32_t bt_s[kBtLds];

    const Item it = work_item(a);
    const Range R = split_range(a, it.seq, it.split);
    const bool direct = a.max_splits == 1;
    if (!direct && R.hi <= R.lo) {  // not a live split (uniform per workgroup)
        if (a.fused_merge && R.len <= 0 && it.split == 0) zero_outputs<DT, D, G>(a, it.seq, it.hg);
        return;
    }
    const int64_t jb0 = stage_table(a, it.seq, R, bt_s);

    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = it.hg * a.heads_per_wg + w;  // < num_kv_heads: head groups tile the heads
    const int r = lane / LPR;
    const int c = lane % LPR;
    const int hq0 = h * G;
    const int seq = it.seq;
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;

    u32x4 qv[G];
    {
        const char *qp = a.q + ((int64_t)seq * a.num_q_heads + hq0) * (D * E) + c * 16;
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g] = ld16(qp + g * (D * E));
    }

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = 0.0f;
    }

    const char *kb = a.pool.k + a.pool.layer_off + (int64_t)h * (D * E) + c * 16;
    const char *vb = a.pool.v + a.pool.layer_off + (int64_t)h * (D * E) + c * 16;

    // Decode with append: the work item that ends the sequence first writes
    // the new token's K/V row (logical position len - 1); each piece is
    // stored by the lane whose load below reads it back.
    if (a.k_new != nullptr && R.whole && R.len > 0 && R.hi == R.off + R.len) {
        const int64_t pn = R.hi - 1;
        if (r == (int)((pn - R.lo) % kChunkTokens) % RPI) {
            const int32_t b = bt_s[(int)((pn >> lbs) - jb0)];
            if (b >= 0) {
                const int64_t src = ((int64_t)seq * a.num_kv_heads + h) * (D * E) + c * 16;
                const int64_t o = (int64_t)b * a.pool.block_stride + (pn & bsm) * a.pool.row_bytes;
                *reinterpret_cast<u32x4 *>(const_cast<char *>(kb) + o) = ld16(a.k_new + src);
                *reinterpret_cast<u32x4 *>(const_cast<char *>(vb) + o) = ld16(a.v_new + src);
            }
        }
    }

    for (int64_t pc = R.lo; pc < R.hi; pc += kChunkTokens) {
        u32x4 kx[NP], vx[NP];
        bool ok[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int64_t p = pc + i * RPI + r;
            ok[i] = false;
            kx[i] = u32x4{0, 0, 0, 0};
            vx[i] = u32x4{0, 0, 0, 0};
            if (p < R.hi) {
                const int32_t b = bt_s[(int)((p >> lbs) - jb0)];
                if (b >= 0) {
                    ok[i] = true;
                    const int64_t o = (int64_t)b * a.pool.block_stride + (p & bsm) * a.pool.row_bytes;
                    kx[i] = ld16(kb + o);
                    vx[i] = ld16(vb + o);
                }
            }
        }

        float s[NP][G];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const float d = row_allsum<LPR>(dot16<DT>(qv[g], kx[i]));
                s[i][g] = ok[i] ? d * a.scale_log2 : kNegInf;
            }
        }

        float p[NP][G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float cm = s[0][g];
#pragma unroll
            for (int i = 1; i < NP; ++i) cm = fmaxf(cm, s[i][g]);
            cm = cross_rows_max<LPR>(cm);
            const float mn = fmaxf(m[g], cm);
            const float alpha = mn == kNegInf ? 1.0f : fast_exp2(m[g] - mn);
            float ps = 0.0f;
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                p[i][g] = s[i][g] == kNegInf ? 0.0f : fast_exp2(s[i][g] - mn);
                ps += p[i][g];
            }
            l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
            for (int e = 0; e < VEC; ++e) acc[g][e] *= alpha;
            m[g] = mn;
        }

#pragma unroll
        for (int i = 0; i < NP; ++i) {
            float vf[VEC];
            unpack16<DT>(vx[i], vf);
#pragma unroll
            for (int g = 0; g < G; ++g) {
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(p[i][g], vf[e], acc[g][e]);
            }
        }
    }

#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = cross_rows_sum<LPR>(l[g]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = cross_rows_sum<LPR>(acc[g][e]);
    }
    if (direct) {
        if (r != 0) return;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = l[g] > 0.0f ? acc[g][e] / l[g] : 0.0f;
            store16<DT>(a.out + (((int64_t)seq * a.num_q_heads + hq0 + g) * D + c * VEC) * E, o);
        }
        return;
    }
    if (r == 0) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t item = ((int64_t)seq * a.max_splits + it.split) * a.num_q_heads + hq0 + g;
            float *wa = a.ws_acc + item * D + c * VEC;
#pragma unroll
            for (int e = 0; e < VEC; e += 2) st_dev2(wa + e, acc[g][e], acc[g][e + 1]);
            if (c == 0) st_dev2(a.ws_ml + item * 2, m[g], l[g]);
        }
    }
    if (a.fused_merge) finish_split<DT, D, G, false>(a, it, R, a.split_tokens);
}

// ---------------------------------------------------------------------------
// bf16 pools: QK^T and P.V both on the matrix core.
// UB: block_size >= 16, so a 16-position chunk lies inside one block and its
// block id is wave-uniform (scalar address arithmetic).
//
// Per 16-position chunk and wavefront (one kv head):
//   Loads: K and V rows are read in "row layout" -- each load instruction
//      moves four whole 256-byte rows (lane (r, c) takes 16-byte piece c of
//      row r), the pattern the L1 and its TLB serve best.  K goes into a
//      register ring, V straight into an LDS ring (global_load_lds_dwordx4),
//      both NSLOT-1 chunks ahead of the chunk being computed.
//   QK^T: the K chunk is written to a per-wave LDS tile and read back in the
//      MFMA A-operand layout (lane l: row l%16, elements 32j + 8*(l/16) ..);
//      S^T (16 tokens x 16 heads) = K . Q^T (heads >= G zero) with
//      v_mfma_f32_16x16x32_bf16.  Lane l then holds the scores of tokens
//      4*(l/16) .. +3 for head l%16.
//   softmax in registers (exp2 domain, lazy reference max); the lane's four
//      probabilities, rounded to bf16, are exactly its A operand for P.V.
//   P.V: the B operand (four consecutive tokens of one column per lane)
//      comes from the V tile with ds_read_b64_tr_b16, the transposing LDS
//      read; O (16 heads x D) += P . V with v_mfma_f32_16x16x16_bf16 per
//      16-column slab; lane l accumulates O[head 4*(l/16) + i][16*slab + l%16].
//   Both tiles are padded so the column-wise operand reads hit distinct LDS
//      banks while every address stays one base register plus constants.
//   Every load is issued unconditionally from an in-bounds address (a
//   missing block reads block 0), so the waits stay exact.  Rows without a
//   live token are zeroed in the V tile (a 0 * NaN product would poison the
//   sum) and get score -inf.

// Q^T fragments of kv head h's G query heads (B operand of QK^T): lane l
// holds head l%16 (zero for heads >= G), elements 32j + 8*(l/16) .. +8.
template <int D, int G>
__device__ __forceinline__ void load_q(const DecodeArgs &a, int seq, int h,
                                       u32x4 (&qf)[MfmaShape<D>::KS]) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
    const char *qp = a.q + (((int64_t)seq * a.num_q_heads + (int64_t)h * G + n) * D + 8 * g4) * 2;
#pragma unroll
    for (int j = 0; j < MfmaShape<D>::KS; ++j) qf[j] = n < G ? ld16(qp + 64 * j) : u32x4{0, 0, 0, 0};
}

// Wait until at most `ahead` chunks' loads (LOADS vector-memory operations
// each) are outstanding: the copy engine's LDS writes of a ring slot are not
// tracked by the compiler, so each compute step waits explicitly.  The count
// is an immediate, hence the switch (ahead < 4).
template <int LOADS>
__device__ __forceinline__ void wait_chunks_in_flight(int ahead) {
    auto w = [](auto c) {
        constexpr int n = decltype(c)::value * LOADS;
        __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
    };
    switch (ahead) {
        case 3: w(std::integral_constant<int, 3>{}); break;
        case 2: w(std::integral_constant<int, 2>{}); break;
        case 1: w(std::integral_constant<int, 1>{}); break;
        default: w(std::integral_constant<int, 0>{}); break;
    }
}

// Attention of one wavefront's kv head h over the flat positions [R.lo, R.hi)
// of one sequence, accumulated into (m_h, l_h, acc): the per-chunk pipeline
// described above.  bt_s holds the table entries from jb0 on.
template <int D, int G, bool UB>
__device__ __forceinline__ void attend_range(const DecodeArgs &a, int seq, const Range &R, int64_t jb0,
                                             const int32_t *bt_s, char *vring, int h,
                                             const u32x4 (&qf)[MfmaShape<D>::KS], float &m_h,
                                             float &l_h, f32x4 (&acc)[MfmaShape<D>::NV]) {
    using S = MfmaShape<D>;
    constexpr int ROWB = S::ROWB, PPR = S::PPR, NP = S::NP, KS = S::KS, NV = S::NV;
    constexpr int VSLAB = S::VSLAB, VTILE = S::VTILE, NSLOT = S::NSLOT;
    constexpr int LOADS = S::LOADS;
    constexpr float kLazy = 8.0f;  // reference-max slack, log2 units
    const int lane = threadIdx.x & 63;
    const int n = lane & 15;       // MFMA: row / column index
    const int g4 = lane >> 4;      // MFMA: k group
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;
    const int64_t row_bytes = a.pool.row_bytes;
    const float sl2 = a.scale_log2;

    const char *kh = a.pool.k + a.pool.layer_off + (int64_t)h * ROWB;
    const char *vh = a.pool.v + a.pool.layer_off + (int64_t)h * ROWB;
    // V row-layout load role: load instruction i moves rows i + NP*q,
    // q = lane / PPR, and this lane takes their 16-byte piece lane % PPR.
    // In the V tile instruction i's 1 KiB lands at slab i (slabs padded so
    // the four rows a P.V operand read touches sit in different banks).
    const int trow = lane / PPR;
    const int tpp = lane % PPR;

    // Issue the loads of chunk pc: K straight into registers in the MFMA
    // A-operand layout (lane (n, g4) takes row n, bytes 64 j + 16 g4 .. +16
    // for step j), V into ring slot `slot` in row layout.
    auto load_chunk = [&](int64_t pc, u32x4 *kx, int slot) {
        char *dst = vring + slot * VTILE;
        if constexpr (UB) {
            int32_t b = __builtin_amdgcn_readfirstlane(bt_s[(int)((pc >> lbs) - jb0)]);
            const int64_t base = (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride + (pc & bsm) * row_bytes;
            const char *kb = kh + base + (uint32_t)(n * row_bytes + 16 * g4);
            const char *vb = vh + base;
#pragma unroll
            for (int j = 0; j < KS; ++j) kx[j] = ld16(kb + 64 * j);
#pragma unroll
            for (int i = 0; i < NP; ++i)
                lds_copy16_nt(vb + (uint32_t)((i + NP * trow) * row_bytes + 16 * tpp), dst + i * VSLAB);
        } else {
            {
                const int64_t p = pc + n;
                const bool in = p >= R.lo && p < R.hi;
                const int32_t b = in ? bt_s[(int)((p >> lbs) - jb0)] : -1;
                const char *kb = kh + (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride + (p & bsm) * row_bytes + 16 * g4;
#pragma unroll
                for (int j = 0; j < KS; ++j) kx[j] = ld16(kb + 64 * j);
            }
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int64_t p = pc + i + NP * trow;
                const bool in = p >= R.lo && p < R.hi;
                const int32_t b = in ? bt_s[(int)((p >> lbs) - jb0)] : -1;
                const int64_t o = (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride + (p & bsm) * row_bytes + 16 * tpp;
                lds_copy16_nt(vh + o, dst + i * VSLAB);
            }
        }
    };
    auto compute = [&](int64_t pc, const u32x4 *kc, int slot, int ahead) {
        // This chunk's loads were issued NSLOT-1 chunks ago; wait for them
        // (the V tile is written by the copy engine, which the compiler does
        // not track) while the `ahead` later chunks' loads stay in flight.
        wait_chunks_in_flight<LOADS>(ahead);
        wave_lds_order();
        char *vt = vring + slot * VTILE;
        // live rows of the chunk: [rlo, rhi) relative to pc (32-bit, wave
        // uniform), and (block size < 16) a table entry per row
        const int64_t dlo = R.lo - pc, dhi = R.hi - pc;
        const int32_t rlo = dlo > 0 ? (int32_t)dlo : 0;
        int32_t rhi = dhi < 16 ? (int32_t)dhi : 16;
        if constexpr (UB) {
            if (__builtin_amdgcn_readfirstlane(bt_s[(int)((pc >> lbs) - jb0)]) < 0) rhi = 0;
        }
        auto row_live = [&](int row) -> bool {
            const bool in = row >= rlo && row < rhi;
            if constexpr (UB) return in;
            else return in && bt_s[(int)(((pc + row) >> lbs) - jb0)] >= 0;
        };
        const bool full = UB ? (rlo == 0 && rhi == 16) : false;
        if (!full) {
            // zero the tile rows that hold no live token
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                if (!row_live(i + NP * trow))
                    *reinterpret_cast<u32x4 *>(vt + i * VSLAB + 16 * lane) = u32x4{0, 0, 0, 0};
            }
            wave_lds_order();
        }
        // scores: lane holds S[token 4*g4 + i][head n]
        f32x4 sacc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int j = 0; j < KS; ++j)
            sacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kc[j]), as_bf16x8(qf[j]), sacc, 0, 0, 0);
        float s[4];
        float cm = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float x = sacc[i] * sl2;
            s[i] = row_live(4 * g4 + i) ? x : kNegInf;
            cm = fmaxf(cm, s[i]);
        }
        cm = max_xor32(max_xor16(cm));
        float alpha = 1.0f;
        if (cm > m_h + kLazy) {
            alpha = m_h == kNegInf ? 0.0f : fast_exp2(m_h - cm);
            m_h = cm;
        }
        float pr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = s[i] == kNegInf ? 0.0f : fast_exp2(s[i] - m_h);
        // P in bf16 (the P.V A operand); the denominator uses the same
        // rounded values
        const uint32_t p01 = bf16x2_rne(pr[0], pr[1]);
        const uint32_t p23 = bf16x2_rne(pr[2], pr[3]);
        l_h = fmaf(l_h, alpha, (bf16_lo(p01) + bf16_hi(p01)) + (bf16_lo(p23) + bf16_hi(p23)));
        if (__any(n < G && alpha != 1.0f)) {
            // rescale O rows (heads 4*g4 + i) by their heads' alpha
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float al = __shfl(alpha, 4 * g4 + i);
#pragma unroll
                for (int sl = 0; sl < NV; ++sl) acc[sl][i] *= al;
            }
        }
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 pa = __builtin_bit_cast(s16x4, (uint64_t)p01 | ((uint64_t)p23 << 32));
        // this lane's operand rows: token 4*g4 + (n >> 2), columns 16*sl + 4*(n&3)
        const int vrow = 4 * g4 + (n >> 2);
        const int vbase = (vrow % NP) * VSLAB + (vrow / NP) * ROWB + 8 * (n & 3);
#pragma unroll
        for (int sl = 0; sl < NV; ++sl) {
            const int off = vbase + 32 * sl;
            const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)(vt) + off));
            acc[sl] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[sl], 0, 0, 0);
        }
        wave_lds_order();
    };

    // Ring of NSLOT stages: while chunk c is computed, chunks c+1 ..
    // c+NSLOT-1 are in flight.  No load is issued past the last chunk (a
    // re-read of it under the nontemporal hint went to HBM again: 16 MB per
    // call on the decode batch); the last steps wait for fewer chunks.  The
    // inner loop is unrolled so ring indices are compile-time constants.
    const int64_t first = R.lo & ~int64_t(15);
    if (first < R.hi) {
        const int64_t last = (R.hi - 1) & ~int64_t(15);
        // Decode with append: the range that ends the sequence first writes
        // the new token's K/V row (logical position len - 1, in chunk
        // `last`) into the pool.  Each 16-byte piece is stored by the lane
        // whose ring load reads it back, before that load in program order,
        // so the load sees it.  The new rows are fetched before the ring's
        // first loads; the store waits only for them, and goes after the
        // first loads unless those already cover chunk `last`.
        // (not when the length or offset was clamped: the write would land on
        // another token's slot)
        const bool app = a.k_new != nullptr && R.whole && R.len > 0 && R.hi == R.off + R.len;
        const int64_t pn = R.hi - 1;
        const int rn = (int)(pn & 15);               // the new row within its chunk
        const bool k_lane = app && n == rn;          // loads K pieces 4 j + g4 of that row
        const bool v_lane = app && trow == rn / NP;  // loads V piece tpp of that row
        const int64_t src = ((int64_t)seq * a.num_kv_heads + h) * ROWB;
        u32x4 kn[KS], vn = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < KS; ++j) kn[j] = k_lane ? ld16(a.k_new + src + 64 * j + 16 * g4) : u32x4{0, 0, 0, 0};
        if (v_lane) vn = ld16(a.v_new + src + 16 * tpp);
        auto store_new = [&]() {
            if (!k_lane && !v_lane) return;
            const int32_t b = bt_s[(int)((pn >> lbs) - jb0)];
            if (b < 0) return;  // no block at that position: nothing to write (its score is masked)
            const int64_t o = (int64_t)b * a.pool.block_stride + (pn & bsm) * row_bytes;
            if (k_lane) {
#pragma unroll
                for (int j = 0; j < KS; ++j)
                    *reinterpret_cast<u32x4 *>(const_cast<char *>(kh) + o + 64 * j + 16 * g4) = kn[j];
            }
            if (v_lane) *reinterpret_cast<u32x4 *>(const_cast<char *>(vh) + o + 16 * tpp) = vn;
        };
        const bool store_early = last - first < 16 * (NSLOT - 1);
        if (store_early) store_new();
        u32x4 kring[NSLOT][KS];
#pragma unroll
        for (int q = 0; q < NSLOT - 1; ++q)
            if (first + 16 * q <= last) load_chunk(first + 16 * q, kring[q], q);
        if (!store_early) store_new();
        bool done = false;
        for (int64_t pc = first; !done;) {
#pragma unroll
            for (int q = 0; q < NSLOT; ++q) {
                if (!done) {
                    const int nq = (q + NSLOT - 1) % NSLOT;
                    const int64_t pn = pc + 16 * (NSLOT - 1);
                    if (pn <= last) load_chunk(pn, kring[nq], nq);
                    compute(pc, kring[q], q, (int)min((int64_t)(NSLOT - 1), (last - pc) >> 4));
                    pc += 16;
                    done = pc > last;
                }
            }
        }
        // drain the copy engine before the tiles are reused
        __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
    }
}

// Denominators: l over the token groups (lane (g4, n) then holds head n's l
// in l_h), and lrow[i] = l of head 4*g4 + i, the head of this lane's O row i.
__device__ __forceinline__ void head_denominators(float &l_h, float (&lrow)[4]) {
    const int g4 = (threadIdx.x & 63) >> 4;
    l_h = sum_xor32(sum_xor16(l_h));  // row swaps: no LDS permute round trip
#pragma unroll
    for (int i = 0; i < 4; ++i) lrow[i] = __shfl(l_h, 4 * g4 + i);
}

// out[seq, h*G + hd, :] = acc / l, rounded to bf16.
template <int D, int G>
__device__ __forceinline__ void write_direct(const DecodeArgs &a, int seq, int h,
                                             const f32x4 (&acc)[MfmaShape<D>::NV], const float (&lrow)[4]) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd < G) {
            uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + ((int64_t)seq * a.num_q_heads + (int64_t)h * G + hd) * D + n;
#pragma unroll
            for (int sl = 0; sl < MfmaShape<D>::NV; ++sl)
                o[16 * sl] = (uint16_t)f32_to_bf16_bits(lrow[i] > 0.0f ? acc[sl][i] / lrow[i] : 0.0f);
        }
    }
}

// Unnormalised partial of the wave's G heads: acc rows at accp + hd*D and
// (m, l) pairs at ml + 2*hd, written with device-scope stores.
template <int D, int G>
__device__ __forceinline__ void write_partial(float *ml, float *accp, const f32x4 (&acc)[MfmaShape<D>::NV],
                                              float m_h, float l_h) {
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd < G) {
            float *wa = accp + hd * D + n;
#pragma unroll
            for (int sl = 0; sl < MfmaShape<D>::NV; ++sl) st_dev(wa + 16 * sl, acc[sl][i]);
        }
    }
    if (g4 == 0 && n < G) st_dev2(ml + 2 * n, m_h, l_h);
}

// Half-precision record from G unscaled acc rows (D floats each, row
// order) in the wave's LDS at lds.  Lane p takes the 8 elements [8p, 8p+8)
// (piece p; 16 lanes per head row, so a 16-lane row of the wavefront holds
// one head row), finds the row's shift with one DPP pass, and stores the
// scaled halves as one 16-byte buffer store with the device-scope cache
// policy of st_dev (sc1: through this XCD's L2).  (m, l) of head n (lane n,
// as the attention loop leaves them) are stored re-referenced by the
// shift of its row.  Their completion is awaited with everything else
// before the split is counted in.
template <int D, int G>
__device__ __forceinline__ void store_record_h(float *ml, uint16_t *rec, const char *lds, float m_h, float l_h) {
    static_assert(D == 128, "half-precision records: head_dim 128");
    constexpr int NPC = G * D / 8;       // pieces of 8 elements
    constexpr int NR = (NPC + 63) / 64;  // pieces per lane: 1 for G <= 4, 2 for G = 8
    constexpr int kSC1 = 16;             // cache-policy bit sc1 of a buffer access
    const int lane = threadIdx.x & 63;
    // (readfirstlane returns a signed int: each half of the address is
    // widened through uint32_t.)
    const uint64_t u = reinterpret_cast<uint64_t>(rec);
    const uint32_t ulo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t uhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void *>(((uint64_t)uhi << 32) | ulo), 0, G * D * 2, 0x00020000);
    int kr[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        const int p = lane + 64 * r;
        const bool valid = NPC % 64 == 0 || p < NPC;  // whole 16-lane rows
        f32x4 x0 = {0.0f, 0.0f, 0.0f, 0.0f}, x1 = x0;
        if (valid) {
            x0 = *reinterpret_cast<const f32x4 *>(lds + 32 * p);
            x1 = *reinterpret_cast<const f32x4 *>(lds + 32 * p + 16);
        }
        float mx = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(finite_abs(x0[e]), finite_abs(x1[e])));
        const int k = rec_shift(row_max16(mx));
        kr[r] = k;
        if (valid) {
            float y[8];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                y[e] = __builtin_amdgcn_ldexpf(x0[e], -k);
                y[4 + e] = __builtin_amdgcn_ldexpf(x1[e], -k);
            }
            const u32x4 v = {f16x2_rne(y[0], y[1]), f16x2_rne(y[2], y[3]), f16x2_rne(y[4], y[5]),
                             f16x2_rne(y[6], y[7])};
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, 16 * p, 0, kSC1);
        }
    }
    // the row of head g is lanes 16 (g % 4) .. of piece g / 4; lane g takes
    // its shift by readlane (no LDS permute round trip)
    int kk = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int kg = __builtin_amdgcn_readlane(kr[g >> 2 < NR ? g >> 2 : 0], 16 * (g & 3));
        kk = lane == g ? kg : kk;
    }
    if (lane < G) st_dev2(ml + 2 * lane, m_h + (float)kk, __builtin_amdgcn_ldexpf(l_h, -kk));
}

// The partial of the P.V output layout as a half-precision record (head_dim
// 128).  Lane (n, g4) holds column n + 16*sl of heads 4*g4 .. 4*g4+3, 4
// bytes from the next lane's: the rows are put in record order in the
// wave's free LDS (G*D floats at lds, no longer used by the attention loop)
// and stored from there.
template <int D, int G>
__device__ __forceinline__ void write_partial_h(float *ml, uint16_t *rec, const f32x4 (&acc)[MfmaShape<D>::NV],
                                                float m_h, float l_h, char *lds) {
    constexpr int NV = MfmaShape<D>::NV;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
    float *t = reinterpret_cast<float *>(lds);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd < G) {
#pragma unroll
            for (int sl = 0; sl < NV; ++sl) t[hd * D + n + 16 * sl] = acc[sl][i];
        }
    }
    wave_lds_order();
    store_record_h<D, G>(ml, rec, lds, m_h, l_h);
    wave_lds_order();
}

// Split schedule: one workgroup per (sequence, split, head group).
template <int D, int G, bool UB>
__global__ __launch_bounds__(256) void decode_mfma_kernel(DecodeArgs a) {
    using S = MfmaShape<D>;
    static_assert(G >= 1 && G <= 16, "group");
    __shared__ int32_t bt_s[kBtLds];
    __shared__ __attribute__((aligned(16))) char vtiles[4][S::NSLOT][S::VTILE];
    static_assert(!kRecordsHalf<D> || G * D * 4 <= S::NSLOT * S::VTILE, "record assembly fits the V ring");

    Item it;
    Range R;
    int64_t split = a.split_tokens;
    bool direct;
    if (a.plan) {
        if (!plan_item<D, G>(a, bt_s, it, R, split)) return;
        direct = R.lo == R.off && R.hi == R.off + R.len;  // the sequence's only piece
    } else {
        it = work_item(a);
        R = split_range(a, it.seq, it.split);
        direct = a.max_splits == 1;
        if (!direct && R.hi <= R.lo) {
            if (a.fused_merge && R.len <= 0 && it.split == 0) zero_outputs<1, D, G>(a, it.seq, it.hg);
            return;
        }
    }
    const int64_t jb0 = stage_table(a, it.seq, R, bt_s);

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = it.hg * a.heads_per_wg + w;  // < num_kv_heads: head groups tile the heads
    u32x4 qf[S::KS];
    load_q<D, G>(a, it.seq, h, qf);
    float m_h = kNegInf;  // reference max of head n (same in its 4 lanes)
    float l_h = 0.0f;     // this lane's share of head n's denominator
    f32x4 acc[S::NV];
#pragma unroll
    for (int sl = 0; sl < S::NV; ++sl) acc[sl] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    attend_range<D, G, UB>(a, it.seq, R, jb0, bt_s, vtiles[w][0], h, qf, m_h, l_h, acc);
    float lrow[4];
    head_denominators(l_h, lrow);
    if (direct) {
        write_direct<D, G>(a, it.seq, h, acc, lrow);
        return;
    }
    const int64_t item0 = ((int64_t)it.seq * a.max_splits + it.split) * a.num_q_heads + (int64_t)h * G;
    // the wave's V ring is free now: it assembles the half-precision record
    // (head_dim 128) or stages merge records (64)
    bool half_rec = false;
    if constexpr (kRecordsHalf<D>) {
        half_rec = a.fused_merge;
        if (half_rec)
            write_partial_h<D, G>(a.ws_ml + item0 * 2, reinterpret_cast<uint16_t *>(a.ws_acc) + item0 * D, acc, m_h,
                                  l_h, vtiles[w][0]);
    }
    if (!half_rec) write_partial<D, G>(a.ws_ml + item0 * 2, a.ws_acc + item0 * D, acc, m_h, l_h);
    if (a.fused_merge)
        finish_split<1, D, G, kRecordsHalf<D>>(a, it, R, split, vtiles[w][0], S::NSLOT * S::VTILE);
}

// ---------------------------------------------------------------------------
// Quantised pools (int8, int4), split schedule [P3 sec. 6 names quantised KV;
// the stored value of a (token, kv head) row is code * scale].  One 16-token
// chunk per step, as decode_mfma_kernel, with the codes' bytes:
//   K: QK^T runs on the int8 matrix cores (v_mfma_i32_16x16x64_i8) on the
//      codes as loaded: lane (n, g4) loads row n's codes [D/4 g4, D/4 (g4+1))
//      and step j (64 codes) takes 16 of them; the query operand holds the
//      same positions of head n, so the exact int32 sums are dot products
//      whatever order the unit adds them in.  The bf16 query is split per
//      head into two int8 parts, q ~ qh * sh + ql * sl (sh = max|q| / 127,
//      sl = sh / 254: |error| <= max|q| / 64516 per element, finer than the
//      bf16 query itself), so a score is
//      (sh * (qh . code_t) + sl * (ql . code_t)) * kscale_t * scale.
//   V: P.V runs on the bf16 matrix cores (v_mfma_f32_16x16x16_bf16).
//      int8: each lane converts 16 codes of a row to bf16 and writes them to
//      the wave's V tile in the bf16 kernel's layout; the product reads the
//      tile with the same transposing LDS read.  int4: the codes are the B
//      operand straight from registers: lane (n, g4) loads columns
//      [C n, C n + C) (C = D / 16) of its four tokens 4 g4 .. 4 g4 + 3, the
//      rows whose probabilities its score lanes already hold, and unpacks
//      them into bf16 operands of 136 + code (see i4_operands); no LDS sits
//      between the loads and the product, and lane (n, g4) accumulates
//      columns [C n, C n + C) of heads 4 g4 .. 4 g4 + 3, so one store
//      instruction of the outputs or partials covers a head row.  The value
//      scale folds into the probabilities: P'_t = p_t * vscale_t (rounded to
//      bf16 as P is); the denominator sums P'_t / vscale_t, the weights the
//      operand carries; int4 subtracts 136 * sum(P') per head at the end.
//   Scales: the 16 tokens of a chunk are contiguous per head (layout
//      (block, layer, head, slot)), so lane (n, g4) loads the scales of its
//      four tokens 4 g4 .. 4 g4 + 3 with one 16-byte load each.
//   int4 K: a nibble moved to the top of its byte is the signed byte
//      16 * code, so the int8 score path applies; the 1/16 goes into the
//      query's scales.
//   Codes are always finite, so rows without a live token need no zeroing:
//   their score is -inf and their P' exactly 0.
// ---------------------------------------------------------------------------

// int4: eight codes in a word (byte k: element 2k in the low nibble, 2k + 1
// in the high nibble) as bytes holding 16 * code, exactly: the nibble moved
// to the top of its byte is a signed byte of 16 * code.  even: elements 0, 2,
// 4, 6; odd: elements 1, 3, 5, 7 (byte k = element 2k or 2k + 1).
__device__ __forceinline__ uint32_t i4_even16(uint32_t w) { return (w << 4) & 0xF0F0F0F0u; }
__device__ __forceinline__ uint32_t i4_odd16(uint32_t w) { return w & 0xF0F0F0F0u; }

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 ld8_nt(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}
__device__ __forceinline__ uint32_t ld4_nt(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint32_t *>(p));
}
__device__ __forceinline__ uint32_t ld2_nt(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const uint16_t *>(p));
}

typedef int v4i32 __attribute__((ext_vector_type(4)));

// The query of head n as int8 operands: lane (n, g4), step j holds the hi
// and lo codes of elements D/4 g4 + 16 j .. +16, and every lane of head n
// the two scales.  Heads >= G are zero.
template <int D>
struct Q8Query {
    static constexpr int KL = D / 64;
    v4i32 hi[KL], lo[KL];
    float sh, sl;
};

__device__ __forceinline__ uint32_t q8_code(float x, float inv) {
    return (uint32_t)(int32_t)fminf(fmaxf(__builtin_rintf(x * inv), -127.0f), 127.0f) & 0xffu;
}

// The bf16 query elements a lane quantises: lane l takes the 8 elements
// 8 (l % LPH) .. +8 of head l / LPH + HPP i in pass i (LPH = D / 8 lanes per
// head, HPP = 64 / LPH heads per pass), so every lane works and a head's
// lanes are one aligned group of a 16-lane row.  Issued before the first
// chunk's loads, so the quantisation runs while those are in flight.
// Lanes past the G heads load head G - 1 (no branch around the loads,
// whose merge would wait for them) and quantise zeros.
template <int D, int G>
struct QRaw {
    static constexpr int LPH = D / 8, HPP = 64 / LPH, NPASS = (G + HPP - 1) / HPP;
    u32x4 w[NPASS];
};

template <int D, int G>
__device__ __forceinline__ void load_q_raw(const DecodeArgs &a, int seq, int h, QRaw<D, G> &raw) {
    using R = QRaw<D, G>;
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < R::NPASS; ++i) {
        const int r = lane / R::LPH + R::HPP * i;
        const int hr = r < G ? r : G - 1;
        raw.w[i] = ld16(a.q + (((int64_t)seq * a.num_q_heads + (int64_t)h * G + hr) * D + 8 * (lane % R::LPH)) * 2);
    }
}

// max over each aligned group of W lanes (W = 8 or 16) of a 16-lane row, in
// every lane of the group (DPP: quad swaps, then the half-row and row mirrors)
template <int W>
__device__ __forceinline__ float lane_group_max(float x) {
    static_assert(W == 8 || W == 16, "group");
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    if constexpr (W == 16) x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return x;
}

// The query in two int8 parts per head: q ~ qh sh + ql sl, sh = max|q| / 127,
// sl = sh / 254, codes round-half-even.  Each lane codes its 8 elements,
// the codes go to the wave's LDS at lds (2 G D + 8 G bytes, free until the
// first chunk is computed) in row order with the heads' (sh, sl), and each
// lane (n, g4) then reads its operand fragment of head n: elements D/4 g4 +
// 16 j .. +16 for step j (heads n >= G: zeros).
// QB = 4 (int4 pool): the K codes arrive as 16 * code with each group of 8
// elements in the order 0, 2, 4, 6, 1, 3, 5, 7 (i4_even16 / i4_odd16), so
// the query's codes take the same order and its scales carry the 1/16.
template <int D, int G, int QB>
__device__ __forceinline__ void quantize_q(const QRaw<D, G> &raw, Q8Query<D> &qq, char *lds) {
    using R = QRaw<D, G>;
    constexpr int KL = D / 64;
    const int lane = threadIdx.x & 63;
    char *hib = lds;
    char *lob = lds + G * D;
    float *scl = reinterpret_cast<float *>(lds + 2 * G * D);
#pragma unroll
    for (int i = 0; i < R::NPASS; ++i) {
        const int r = lane / R::LPH + R::HPP * i;
        const bool live = r < G;
        float x[8];
        unpack16<1>(live ? raw.w[i] : u32x4{0, 0, 0, 0}, x);
        float am = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(x[e]));
        const float amax = lane_group_max<R::LPH>(am);
        const float sh = amax / 127.0f;
        const float sl = sh / 254.0f;
        const float ih = amax > 0.0f ? 1.0f / sh : 0.0f;
        const float il = amax > 0.0f ? 1.0f / sl : 0.0f;
        uint32_t wh[2] = {0, 0}, wl[2] = {0, 0};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint32_t ch = q8_code(x[e], ih);
            const float rr = x[e] - (float)(int32_t)(int8_t)ch * sh;
            const int wi = QB == 8 ? e >> 2 : e & 1;
            const int bi = QB == 8 ? e & 3 : e >> 1;
            wh[wi] |= ch << (8 * bi);
            wl[wi] |= q8_code(rr, il) << (8 * bi);
        }
        if (live) {
            const int off = r * D + 8 * (lane % R::LPH);
            *reinterpret_cast<u32x2 *>(hib + off) = u32x2{wh[0], wh[1]};
            *reinterpret_cast<u32x2 *>(lob + off) = u32x2{wl[0], wl[1]};
            if (lane % R::LPH == 0) *reinterpret_cast<f32x2 *>(scl + 2 * r) = f32x2{sh, sl};
        }
    }
    wave_lds_order();
    const int n = lane & 15, g4 = lane >> 4;
    const int hn = n < G ? n : G - 1;
    const v4i32 z = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < KL; ++j) {
        const int off = hn * D + (D / 4) * g4 + 16 * j;
        const v4i32 h4 = *reinterpret_cast<const v4i32 *>(hib + off);
        const v4i32 l4 = *reinterpret_cast<const v4i32 *>(lob + off);
        qq.hi[j] = n < G ? h4 : z;
        qq.lo[j] = n < G ? l4 : z;
    }
    const f32x2 s2 = *reinterpret_cast<const f32x2 *>(scl + 2 * hn);
    qq.sh = QB == 8 ? s2[0] : s2[0] * 0.0625f;
    qq.sl = QB == 8 ? s2[1] : s2[1] * 0.0625f;
    wave_lds_order();  // the tile is written again once the first chunk is computed
}

// int8 V: two codes (bytes sh/8, sh/8 + 1 of w) as a bf16 pair, the high
// halves of their exact float values; 16 codes -> 16 bf16 values (two
// 16-byte pieces, in order).
__device__ __forceinline__ uint32_t i8pair_bf16(uint32_t w, int sh) {
    const float lo = (float)(int32_t)(int8_t)(w >> sh);
    const float hi = (float)(int32_t)(int8_t)(w >> (sh + 8));
    return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}
__device__ __forceinline__ void i8x16_bf16(u32x4 c, u32x4 &lo, u32x4 &hi) {
    lo = u32x4{i8pair_bf16(c.x, 0), i8pair_bf16(c.x, 16), i8pair_bf16(c.y, 0), i8pair_bf16(c.y, 16)};
    hi = u32x4{i8pair_bf16(c.z, 0), i8pair_bf16(c.z, 16), i8pair_bf16(c.w, 0), i8pair_bf16(c.w, 16)};
}

// int4 V: the B operands of columns C n + 2k and C n + 2k + 1 for the
// lane's four rows, as bf16 of kI4Bias + code, two rows per register.  A
// nibble XOR 8 is code + 8 in [0, 15]; OR-ed into the mantissa of bf16 128
// (0x4300) it is the bf16 value 128 + code + 8, exactly.  b[r] is row r's
// code word XOR 0x88888888; one byte permute gathers byte k of two rows (the
// low and the high nibble are columns 2k and 2k + 1), one AND-OR per column
// makes the pair.
constexpr float kI4Bias = 136.0f;
// kM = 0x000F000F and kOne = 0x43004300 come in registers (see the caller).
__device__ __forceinline__ void i4_operands(const uint32_t (&b)[4], int k, uint32_t kM, uint32_t kOne,
                                            uint64_t &even, uint64_t &odd) {
    // byte k of b[r0] to byte 0, byte k of b[r1] to byte 2, zeros elsewhere
    const uint32_t sel = (uint32_t)k | (0x0cu << 8) | ((uint32_t)(4 + k) << 16) | (0x0cu << 24);
    const uint32_t p01 = __builtin_amdgcn_perm(b[1], b[0], sel);
    const uint32_t p23 = __builtin_amdgcn_perm(b[3], b[2], sel);
    even = (uint64_t)((p01 & kM) | kOne) | ((uint64_t)((p23 & kM) | kOne) << 32);
    odd = (uint64_t)(((p01 >> 4) & kM) | kOne) | ((uint64_t)(((p23 >> 4) & kM) | kOne) << 32);
}

// One chunk's loads.  int8: K, the lane's D/4 codes of row n (D/64 16-byte
// loads); V, D/64 16-byte pieces of tile rows (lane: codes 16 (lane % (D/16))
// .. + 16 of row i (64 / (D/16)) + lane / (D/16)).  int4: K, the lane's D/8
// bytes of row n; V, the lane's C = D/16 columns [C n, C n + C) of each of
// its four rows 4 g4 .. 4 g4 + 3, C/2 bytes each.  Both: the K and V scales
// of tokens 4 g4 .. 4 g4 + 3.
template <int D, int QB>
struct QSlot {
    static constexpr int KL = D / 64;
    u32x4 k[KL];
    u32x4 v[D / 64];
    u32x4 ks, vs;
};
template <int D>
struct QSlot<D, 4> {
    u32x4 k;                                 // head_dim 64: .x, .y only
    uint32_t v[4];
    u32x4 ks, vs;
};

// QB: bits per code, 8 (int8 pool: V through the wave's LDS tile, in the
// bf16 kernel's layout) or 4 (int4 pool: V as a register operand).
template <int D, int G, bool UB, int QB>
__device__ __forceinline__ void attend_range_q8(const DecodeArgs &a, const Range &R, int64_t jb0,
                                                const int32_t *bt_s, char *vt, int h,
                                                const QRaw<D, G> &qraw, float &m_h,
                                                float &l_h, float &p_h, f32x4 (&acc)[D / 16]) {
    using S = MfmaShape<D>;
    using Slot = QSlot<D, QB>;
    constexpr int HB = D * QB / 8;   // bytes of one (token, kv head) row of codes
    constexpr int KB = D * QB / 32;  // K code bytes per lane per chunk
    constexpr int C = D / 16;        // P.V column slabs (int4: V columns per lane)
    constexpr int NP = S::NP, ROWB = S::ROWB, VSLAB = S::VSLAB;
    // two slots (one chunk in flight while one is computed): measured
    // faster than three on the decode batch (30.8 against 32.0 us, same
    // process), level on the other batches
    constexpr int NSLOT = 2;
    constexpr int VPR = D / 16;      // int8: 16-code pieces per row
    constexpr int VRPL = 64 / VPR;   // int8: rows per V load
    constexpr float kLazy = 8.0f;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;
    const int64_t row_bytes = a.pool.row_bytes;
    const float sl2 = a.scale_log2;
    Q8Query<D> qq;
    // int4 operand constants, held in registers for the whole range: an
    // AND-OR of three registers is one VOP3 instruction, and VOP3 takes no
    // 32-bit literal on this target (the empty asm keeps them from being
    // folded back into literals)
    uint32_t kI4M = 0x000F000Fu, kI4One = 0x43004300u;
    if constexpr (QB == 4) asm("" : "+v"(kI4M), "+v"(kI4One));
    const char *kh = a.pool.k + a.pool.layer_off + (int64_t)h * HB;
    const char *vh = a.pool.v + a.pool.layer_off + (int64_t)h * HB;
    const float *ksh = a.pool.ks + ((int64_t)h << lbs);
    const float *vsh = a.pool.vs + ((int64_t)h << lbs);
    const int vrow = lane / VPR, vpc = lane % VPR;
    auto load_k = [&](const char *kb, Slot &sl) {
        if constexpr (QB == 8) {
#pragma unroll
            for (int i = 0; i < Slot::KL; ++i) sl.k[i] = ld16_nt(kb + 16 * i);
        } else if constexpr (KB == 16) {
            sl.k = ld16_nt(kb);
        } else {
            const u32x2 w = ld8_nt(kb);
            sl.k = u32x4{w.x, w.y, 0u, 0u};
        }
    };
    // int4 V row r of the lane: C/2 bytes at column C n
    auto load_v4 = [&](const char *row, Slot &sl, int r) {
        if constexpr (D == 128) sl.v[r] = ld4_nt(row + 4 * n);
        else sl.v[r] = ld2_nt(row + 2 * n);
    };

    // int4, whole-block chunks: each chunk's codes and scales are read
    // through buffer resources built from the chunk's (wave-uniform) base
    // addresses, with loop-invariant 32-bit lane offsets, so the loop keeps
    // no 64-bit address temporaries (one of them, reusing a load's
    // destination, made the compiler wait for every load in flight at the
    // top of the loop).  Same process: int4 prefix sharing 48.2 -> 47.4 us,
    // long context 75.0 -> 73.4 us, decode batch level.  int8 measured slower
    // that way (decode batch 24.1 -> 25.05 us, long context 98.2 -> 104.3
    // us) and keeps global loads.
    constexpr int kNT = 2;  // cache-policy bit nt of a buffer access (as ld16_nt)
    const uint32_t koff = (uint32_t)(n * row_bytes + KB * g4);
    auto chunk_rsrc = [](const void *p) {
        // (readfirstlane returns a signed int: each half is widened through
        // uint32_t.)
        const uint64_t u = reinterpret_cast<uint64_t>(p);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
        return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(((uint64_t)hi << 32) | lo), 0,
                                                 0x7fffffff, 0x00020000);
    };
    auto load_chunk = [&](int64_t pc, Slot &sl) {
        if constexpr (UB && QB == 4) {
            const int32_t b = __builtin_amdgcn_readfirstlane(bt_s[(int)((pc >> lbs) - jb0)]);
            const int64_t bb = b >= 0 ? b : 0;
            const int64_t base = bb * a.pool.block_stride + (pc & bsm) * row_bytes;
            const int64_t so = bb * a.pool.sc_block + (pc & bsm);
            const auto rk = chunk_rsrc(kh + base), rv = chunk_rsrc(vh + base);
            const auto rks = chunk_rsrc(ksh + so), rvs = chunk_rsrc(vsh + so);
            if constexpr (KB == 16) {
                sl.k = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, koff, 0, kNT));
            } else {
                const u32x2 w = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rk, koff, 0, kNT));
                sl.k = u32x4{w.x, w.y, 0u, 0u};
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const uint32_t vo = (uint32_t)((4 * g4 + r) * row_bytes);
                if constexpr (D == 128) sl.v[r] = __builtin_amdgcn_raw_buffer_load_b32(rv, vo + 4 * n, 0, kNT);
                else sl.v[r] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rv, vo + 2 * n, 0, kNT);
            }
            sl.ks = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rks, 16 * g4, 0, kNT));
            sl.vs = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rvs, 16 * g4, 0, kNT));
        } else if constexpr (UB) {
            const int32_t b = __builtin_amdgcn_readfirstlane(bt_s[(int)((pc >> lbs) - jb0)]);
            const int64_t bb = b >= 0 ? b : 0;
            const int64_t base = bb * a.pool.block_stride + (pc & bsm) * row_bytes;
            load_k(kh + base + (uint32_t)(n * row_bytes + KB * g4), sl);
#pragma unroll
            for (int i = 0; i < D / 64; ++i)
                sl.v[i] = ld16_nt(vh + base + (uint32_t)((i * VRPL + vrow) * row_bytes + 16 * vpc));
            const int64_t so = bb * a.pool.sc_block + (pc & bsm) + 4 * g4;
            sl.ks = ld16_nt(reinterpret_cast<const char *>(ksh + so));
            sl.vs = ld16_nt(reinterpret_cast<const char *>(vsh + so));
        } else {
            auto row_at = [&](int64_t p, int64_t &bb) {
                const bool in = p >= R.lo && p < R.hi;
                const int32_t b = in ? bt_s[(int)((p >> lbs) - jb0)] : -1;
                bb = b >= 0 ? b : 0;
                return bb * a.pool.block_stride + (p & bsm) * row_bytes;
            };
            int64_t bb;
            load_k(kh + row_at(pc + n, bb) + KB * g4, sl);
            if constexpr (QB == 8) {
#pragma unroll
                for (int i = 0; i < D / 64; ++i)
                    sl.v[i] = ld16_nt(vh + row_at(pc + i * VRPL + vrow, bb) + 16 * vpc);
            }
            uint32_t kw[4], vw[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t p = pc + 4 * g4 + r;
                const int64_t off = row_at(p, bb);
                if constexpr (QB == 4) load_v4(vh + off, sl, r);
                const int64_t so = bb * a.pool.sc_block + (p & bsm);
                kw[r] = __float_as_uint(ksh[so]);
                vw[r] = __float_as_uint(vsh[so]);
            }
            sl.ks = u32x4{kw[0], kw[1], kw[2], kw[3]};
            sl.vs = u32x4{vw[0], vw[1], vw[2], vw[3]};
        }
    };

    auto compute = [&](int64_t pc, const Slot &sl) {
        // live rows of the chunk: [rlo, rhi) relative to pc (32-bit, wave
        // uniform), and (block size < 16) a table entry per row
        const int64_t dlo = R.lo - pc, dhi = R.hi - pc;
        const int32_t rlo = dlo > 0 ? (int32_t)dlo : 0;
        int32_t rhi = dhi < 16 ? (int32_t)dhi : 16;
        if constexpr (UB) {
            if (__builtin_amdgcn_readfirstlane(bt_s[(int)((pc >> lbs) - jb0)]) < 0) rhi = 0;
        }
        auto row_live = [&](int row) -> bool {
            const bool in = row >= rlo && row < rhi;
            if constexpr (UB) return in;
            else return in && bt_s[(int)(((pc + row) >> lbs) - jb0)] >= 0;
        };
        if constexpr (QB == 8) {
            // V codes -> bf16 rows of the tile (the bf16 kernel's slab layout)
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const int row = i * VRPL + vrow;
                u32x4 lo, hi;
                i8x16_bf16(sl.v[i], lo, hi);
                char *dst = vt + (row % NP) * VSLAB + (row / NP) * ROWB + 32 * vpc;
                *reinterpret_cast<u32x4 *>(dst) = lo;
                *reinterpret_cast<u32x4 *>(dst + 16) = hi;
            }
        }
        // scores S[token 4 g4 + i][head n] from the codes as loaded
        v4i32 dh = {0, 0, 0, 0}, dl = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < D / 64; ++j) {
            v4i32 kc;
            if constexpr (QB == 8) {
                kc = __builtin_bit_cast(v4i32, sl.k[j]);
            } else {
                // words 2j, 2j + 1: elements 16j .. 16j + 15 of the lane's
                // range, each group of 8 unpacked as 0, 2, 4, 6, 1, 3, 5, 7
                const uint32_t w0 = j ? sl.k.z : sl.k.x, w1 = j ? sl.k.w : sl.k.y;
                kc = v4i32{(int)i4_even16(w0), (int)i4_odd16(w0), (int)i4_even16(w1), (int)i4_odd16(w1)};
            }
            dh = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, qq.hi[j], dh, 0, 0, 0);
            dl = __builtin_amdgcn_mfma_i32_16x16x64_i8(kc, qq.lo[j], dl, 0, 0, 0);
        }
        const float ksf[4] = {__uint_as_float(sl.ks.x), __uint_as_float(sl.ks.y),
                              __uint_as_float(sl.ks.z), __uint_as_float(sl.ks.w)};
        const float vsf[4] = {__uint_as_float(sl.vs.x), __uint_as_float(sl.vs.y), __uint_as_float(sl.vs.z),
                              __uint_as_float(sl.vs.w)};
        float s[4];
        float cm = kNegInf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float dot = fmaf((float)dh[i], qq.sh, (float)dl[i] * qq.sl);
            const float x = dot * ksf[i] * sl2;
            s[i] = row_live(4 * g4 + i) ? x : kNegInf;
            cm = fmaxf(cm, s[i]);
        }
        cm = max_xor32(max_xor16(cm));
        float alpha = 1.0f;
        if (cm > m_h + kLazy) {
            alpha = m_h == kNegInf ? 0.0f : fast_exp2(m_h - cm);
            m_h = cm;
        }
        float pr[4], pv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            pr[i] = s[i] == kNegInf ? 0.0f : fast_exp2(s[i] - m_h);
            pv[i] = s[i] == kNegInf ? 0.0f : pr[i] * vsf[i];
        }
        const uint32_t q01 = bf16x2_rne(pv[0], pv[1]);
        const uint32_t q23 = bf16x2_rne(pv[2], pv[3]);
        // The denominator sums the weights the P.V operand actually carries,
        // bf16(p * vscale) / vscale, so the output is a convex combination of
        // the stored values code * vscale and a dominant token's rounding
        // cancels (summing bf16(p) instead left up to 2^-8 relative error on
        // peaked rows).  A zero (or tiny) scale is a zero row: its weight is
        // p.
        const float qv[4] = {bf16_lo(q01), bf16_hi(q01), bf16_lo(q23), bf16_hi(q23)};
        float dsum = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) dsum += vsf[i] > 1e-30f ? qv[i] * __builtin_amdgcn_rcpf(vsf[i]) : pr[i];
        l_h = fmaf(l_h, alpha, dsum);
        // int4: the sum of P' the products carry, for the bias kI4Bias * sum
        if constexpr (QB == 4) p_h = fmaf(p_h, alpha, (qv[0] + qv[1]) + (qv[2] + qv[3]));
        if (__any(n < G && alpha != 1.0f)) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float al = __shfl(alpha, 4 * g4 + i);
#pragma unroll
                for (int c = 0; c < C; ++c) acc[c][i] *= al;
            }
        }
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 pa = __builtin_bit_cast(s16x4, (uint64_t)q01 | ((uint64_t)q23 << 32));
        if constexpr (QB == 8) {
            wave_lds_order();
            const int orow = 4 * g4 + (n >> 2);
            const int vbase = (orow % NP) * VSLAB + (orow / NP) * ROWB + 8 * (n & 3);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) s16x4 *)((__attribute__((address_space(3))) char *)(vt) +
                                                                 vbase + 32 * c));
                acc[c] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, vb, acc[c], 0, 0, 0);
            }
            wave_lds_order();
        } else {
            uint32_t b[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = sl.v[r] ^ 0x88888888u;
#pragma unroll
            for (int k = 0; k < C / 2; ++k) {
                uint64_t ev, od;
                i4_operands(b, k, kI4M, kI4One, ev, od);
                acc[2 * k] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, ev),
                                                                       acc[2 * k], 0, 0, 0);
                acc[2 * k + 1] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(pa, __builtin_bit_cast(s16x4, od),
                                                                           acc[2 * k + 1], 0, 0, 0);
            }
        }
    };

    const int64_t first = R.lo & ~int64_t(15);
    if (first < R.hi) {
        const int64_t last = (R.hi - 1) & ~int64_t(15);
        Slot ring[NSLOT];
#pragma unroll
        // Prefetches past the last chunk re-read it, so every step issues
        // the same loads: skipping them instead (a conditional load into the
        // ring registers) made the compiler's waits conservative, measured
        // 67 -> 75 us on prefix sharing.
        for (int q = 0; q < NSLOT - 1; ++q) load_chunk(min(first + 16 * q, last), ring[q]);
        // the query's int8 parts, while the first chunk is in flight (the
        // barrier keeps the scheduler from hoisting them above its loads)
        __builtin_amdgcn_sched_barrier(0);
        quantize_q<D, G, QB>(qraw, qq, vt);
        bool done = false;
        for (int64_t pc = first; !done;) {
#pragma unroll
            for (int q = 0; q < NSLOT; ++q) {
                if (!done) {
                    load_chunk(min(pc + 16 * (NSLOT - 1), last), ring[(q + NSLOT - 1) % NSLOT]);
                    compute(pc, ring[q]);
                    pc += 16;
                    done = pc > last;
                }
            }
        }
    }
}

// int4 path: lane (n, g4) holds columns C n .. C n + C - 1 (C = D / 16) of
// head 4 g4 + i in acc[0..C)[i].  out[seq, h*G + hd, :] = acc / l, rounded
// to bf16: one store of the lane's C columns per head.
template <int D, int G>
__device__ __forceinline__ void write_direct_i4(const DecodeArgs &a, int seq, int h,
                                                const f32x4 (&acc)[D / 16], const float (&lrow)[4]) {
    constexpr int C = D / 16;
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd >= G) continue;
        const float l = lrow[i];
        uint32_t w[C / 2];
#pragma unroll
        for (int c = 0; c < C; c += 2)
            w[c / 2] = bf16x2_rne(l > 0.0f ? acc[c][i] / l : 0.0f, l > 0.0f ? acc[c + 1][i] / l : 0.0f);
        char *o = a.out + (((int64_t)seq * a.num_q_heads + (int64_t)h * G + hd) * D + C * n) * 2;
        if constexpr (C == 8) *reinterpret_cast<u32x4 *>(o) = u32x4{w[0], w[1], w[2], w[3]};
        else *reinterpret_cast<u32x2 *>(o) = u32x2{w[0], w[1]};
    }
}

// int4 path: the unnormalised partial of the wave's G heads, acc rows at
// accp + hd*D and (m, l) pairs at ml + 2*hd.  The acc rows go out as 16-byte
// buffer stores with the device-scope cache policy of st_dev (sc1: through
// this XCD's L2), bounds-checked by the resource to the G rows; their
// completion is awaited with everything else before the split is counted in.
template <int D, int G>
__device__ __forceinline__ void write_partial_i4(float *ml, float *accp, const f32x4 (&acc)[D / 16],
                                                 float m_h, float l_h) {
    constexpr int C = D / 16;
    constexpr int kSC1 = 16;  // cache-policy bit sc1 of a buffer access
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
    // accp is the same in every lane; the resource takes it from SGPRs.
    // (readfirstlane returns a signed int: each half is widened through
    // uint32_t, or a low half with bit 31 set would sign-extend into the
    // high half.)
    const uint64_t u = reinterpret_cast<uint64_t>(accp);
    const uint32_t ulo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t uhi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    float *base = reinterpret_cast<float *>(((uint64_t)uhi << 32) | ulo);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, 0, G * D * 4, 0x00020000);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd >= G) continue;
#pragma unroll
        for (int c = 0; c < C; c += 4) {
            const u32x4 v = {__float_as_uint(acc[c][i]), __float_as_uint(acc[c + 1][i]),
                             __float_as_uint(acc[c + 2][i]), __float_as_uint(acc[c + 3][i])};
            __builtin_amdgcn_raw_buffer_store_b128(v, rs, (hd * D + C * n + c) * 4, 0, kSC1);
        }
    }
    if (g4 == 0 && n < G) st_dev2(ml + 2 * n, m_h, l_h);
}

// int4 path, half-precision record (head_dim 128): lane (n, g4) holds the
// C = 8 contiguous columns C*n .. C*n+7 of heads 4*g4 .. 4*g4+3; the rows go
// to the wave's free LDS (G*D floats at lds) in two 16-byte writes per
// head and are stored from there.
template <int D, int G>
__device__ __forceinline__ void write_partial_i4_h(float *ml, uint16_t *rec, const f32x4 (&acc)[D / 16],
                                                   float m_h, float l_h, char *lds) {
    constexpr int C = D / 16;
    static_assert(C == 8, "half-precision records: head_dim 128");
    const int lane = threadIdx.x & 63;
    const int n = lane & 15, g4 = lane >> 4;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int hd = 4 * g4 + i;
        if (hd < G) {
            f32x4 *t = reinterpret_cast<f32x4 *>(lds + (hd * D + C * n) * 4);
            t[0] = f32x4{acc[0][i], acc[1][i], acc[2][i], acc[3][i]};
            t[1] = f32x4{acc[4][i], acc[5][i], acc[6][i], acc[7][i]};
        }
    }
    wave_lds_order();
    store_record_h<D, G>(ml, rec, lds, m_h, l_h);
    wave_lds_order();
}

// QB: bits per code of the pool, 8 or 4.
template <int D, int G, bool UB, int QB>
// Two wavefronts per SIMD: without the hint the compiler takes 272
// registers (one wavefront per SIMD, half the loads in flight).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void decode_q8_kernel(DecodeArgs a) {
    using S = MfmaShape<D>;
    static_assert(G >= 1 && G <= 16, "group");
    __shared__ int32_t bt_s[kBtLds];
    // int8: the wave's V tile; both: merge records of the fused merge
    __shared__ __attribute__((aligned(16))) char vtiles[4][S::VTILE];
    static_assert(!kRecordsHalf<D> || G * D * 4 <= S::VTILE, "record assembly fits the V tile");
    static_assert(2 * G * D + 8 * G <= S::VTILE, "the query's codes fit the V tile");

    Item it;
    Range R;
    int64_t split = a.split_tokens;
    bool direct;
    if (a.plan) {
        if (!plan_item<D, G>(a, bt_s, it, R, split)) return;
        direct = R.lo == R.off && R.hi == R.off + R.len;  // the sequence's only piece
    } else {
        it = work_item(a);
        R = split_range(a, it.seq, it.split);
        direct = a.max_splits == 1;
        if (!direct && R.hi <= R.lo) {
            if (a.fused_merge && R.len <= 0 && it.split == 0) zero_outputs<1, D, G>(a, it.seq, it.hg);
            return;
        }
    }
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int h = it.hg * a.heads_per_wg + w;
    // the query's loads go out before the table's, so it has arrived by the
    // time the first chunk's loads are issued and its quantisation starts
    QRaw<D, G> qraw;
    load_q_raw<D, G>(a, it.seq, h, qraw);
    const int64_t jb0 = stage_table(a, it.seq, R, bt_s);
    float m_h = kNegInf;
    float l_h = 0.0f;
    float p_h = 0.0f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int c = 0; c < D / 16; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    attend_range_q8<D, G, UB, QB>(a, R, jb0, bt_s, vtiles[w], h, qraw, m_h, l_h, p_h, acc);
    float lrow[4];
    head_denominators(l_h, lrow);
    if constexpr (QB == 4) {
        // remove the operand bias: acc row i (head 4 g4 + i) minus
        // kI4Bias * (sum of that head's P'), before the partials or outputs
        float prow[4];
        head_denominators(p_h, prow);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int c = 0; c < D / 16; ++c) acc[c][i] = fmaf(-kI4Bias, prow[i], acc[c][i]);
    }
    const int64_t item0 = ((int64_t)it.seq * a.max_splits + it.split) * a.num_q_heads + (int64_t)h * G;
    uint16_t *rec = reinterpret_cast<uint16_t *>(a.ws_acc) + item0 * D;
    if constexpr (QB == 8) {
        if (direct) {
            write_direct<D, G>(a, it.seq, h, acc, lrow);
            return;
        }
        // the wave's V tile is free now
        bool half_rec = false;
        if constexpr (kRecordsHalf<D>) {
            half_rec = a.fused_merge;
            if (half_rec) write_partial_h<D, G>(a.ws_ml + item0 * 2, rec, acc, m_h, l_h, vtiles[w]);
        }
        if (!half_rec) write_partial<D, G>(a.ws_ml + item0 * 2, a.ws_acc + item0 * D, acc, m_h, l_h);
    } else {
        if (direct) {
            write_direct_i4<D, G>(a, it.seq, h, acc, lrow);
            return;
        }
        bool half_rec = false;
        if constexpr (kRecordsHalf<D>) {
            half_rec = a.fused_merge;
            if (half_rec) write_partial_i4_h<D, G>(a.ws_ml + item0 * 2, rec, acc, m_h, l_h, vtiles[w]);
        }
        if (!half_rec) write_partial_i4<D, G>(a.ws_ml + item0 * 2, a.ws_acc + item0 * D, acc, m_h, l_h);
    }
    if (a.fused_merge) finish_split<1, D, G, kRecordsHalf<D>>(a, it, R, split, vtiles[w], S::VTILE);
}

// ---------------------------------------------------------------------------
// Merge kernel, used when sequences span many splits: merge the live
// splits of one (sequence, query head):
//   M = max_j m_j,  w_j = 2^(m_j - M),  L = sum_j l_j w_j,
//   out = (sum_j w_j acc_j) / L.
// One 256-thread workgroup per (sequence, query head).  The split weights
// are computed once into LDS; thread t then owns output element t % D and
// the splits j = t / D, t / D + NG, ... (NG = 256 / D groups), with its
// loads unrolled so many are in flight; the NG group sums are added in
// group order through LDS.  The partition is fixed, so results are
// bitwise reproducible.
// ---------------------------------------------------------------------------
constexpr int kReduceThreads = 256;

template <int DT, int D>
__global__ __launch_bounds__(kReduceThreads) void reduce_kernel(DecodeArgs a) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int NG = kReduceThreads / D;  // split groups
    constexpr int U = 16;                   // acc values per thread in the first batch
    static_assert(NG >= 1 && kReduceThreads % D == 0, "head_dim");
    extern __shared__ float w_s[];          // max_splits weights
    __shared__ float red_s[kReduceThreads / 64];
    __shared__ float part_s[NG][D];

    const int seq = blockIdx.x / a.num_q_heads;
    const int hq = blockIdx.x - seq * a.num_q_heads;
    const int64_t item0 = (int64_t)seq * a.max_splits * a.num_q_heads + hq;
    const int64_t step = a.num_q_heads;
    const int ns = a.max_splits;
    const int t = threadIdx.x;
    const int wv = t >> 6;
    const int d = t % D;
    const int grp = t / D;
    const float *src = a.ws_acc + item0 * D + d;
    const int64_t jstride = step * D;

    // One memory round trip for the common case: the length and offset,
    // the (m, l) of splits t (< kReduceThreads) and this thread's first U
    // acc values (splits grp, grp + NG, ...), all loaded before any is
    // used.  Records of empty splits hold stale values; they are loaded
    // (the workspace holds every split) and get weight 0.
    int64_t L = a.seq_lens[seq];
    int64_t off = a.offsets[seq];
    bool whole;
    clamp_len_off(a, L, off, whole);
    float2 ml0 = make_float2(kNegInf, 0.0f);
    if (t < ns) ml0 = *reinterpret_cast<const float2 *>(a.ws_ml + (item0 + t * step) * 2);
    float x0[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = grp + u * NG;
        x0[u] = j < ns ? src[(int64_t)j * jstride] : 0.0f;
    }
    const int64_t S = a.split_tokens;
    auto live = [&](int j) {  // split j holds tokens: [jS, (j+1)S) meets [off, off + L)
        return max((int64_t)j * S, off) < min((int64_t)(j + 1) * S, off + L);
    };

    // 1. max over live splits
    float M = t < ns && live(t) ? ml0.x : kNegInf;
    for (int j = t + kReduceThreads; j < ns; j += kReduceThreads)
        if (live(j)) M = fmaxf(M, a.ws_ml[(item0 + j * step) * 2]);
    M = wave_max(M);  // DPP and row swaps: no LDS permute round trips
    if ((t & 63) == 0) red_s[wv] = M;
    __syncthreads();
    M = red_s[0];
#pragma unroll
    for (int k = 1; k < kReduceThreads / 64; ++k) M = fmaxf(M, red_s[k]);
    __syncthreads();
    // 2. weights and denominator
    float den = 0.0f;
    for (int j = t; j < ns; j += kReduceThreads) {
        float wj = 0.0f;
        if (live(j)) {
            const float2 ml = j == t ? ml0 : *reinterpret_cast<const float2 *>(a.ws_ml + (item0 + j * step) * 2);
            wj = ml.x == kNegInf ? 0.0f : fast_exp2(ml.x - M);
            den = fmaf(ml.y, wj, den);
        }
        w_s[j] = wj;
    }
    den = wave_sum(den);  // a fixed order, so the result does not depend on timing
    if ((t & 63) == 0) red_s[wv] = den;
    __syncthreads();
    den = red_s[0];
#pragma unroll
    for (int k = 1; k < kReduceThreads / 64; ++k) den += red_s[k];

    // 3. weighted sum of this thread's splits for element d, in split order
    float o = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = grp + u * NG;
        if (j < ns) {
            const float wj = w_s[j];
            o = fmaf(wj != 0.0f ? x0[u] : 0.0f, wj, o);
        }
    }
    for (int j = grp + U * NG; j < ns; j += NG) {
        const float wj = w_s[j];
        const float x = src[(int64_t)j * jstride];
        o = fmaf(wj != 0.0f ? x : 0.0f, wj, o);
    }
    part_s[grp][d] = o;
    __syncthreads();
    if (grp == 0) {
        float tot = part_s[0][d];
#pragma unroll
        for (int g = 1; g < NG; ++g) tot += part_s[g][d];
        const float v = den > 0.0f ? tot / den : 0.0f;
        char *dst = a.out + (((int64_t)seq * a.num_q_heads + hq) * D + d) * E;
        if constexpr (DT == 1) {
            *reinterpret_cast<uint16_t *>(dst) = (uint16_t)f32_to_bf16_bits(v);
        } else {
            *reinterpret_cast<float *>(dst) = v;
        }
    }
}

// ---------------------------------------------------------------------------
// The bf16 decode kernels at head_dim 128 with G <= 4 are built in a second
// object from this file (PKV_DECODE_ACC_VGPR, compiled with LLVM's
// -amdgpu-mfma-vgpr-form), so their matrix-core accumulators live in
// ordinary vector registers.  In AGPRs they are copied into vector
// registers at the top of each ring iteration, some of which pending ring
// loads still target, so the compiler waited for every load in flight
// there.  Same process: decode batch 35.45 -> 34.95 us, prefix sharing 89.6
// -> 88.9 us.  The G = 8 kernel (long context) measured slower that way
// (167.3 -> 169.4 us) and stays in this object.  Each kernel instance is
// built in exactly one of the two objects.
// ---------------------------------------------------------------------------
template <int D, int G>
constexpr bool kAccVgprObject = D == 128 && G <= 4;

hipError_t launch_decode_mfma_vgpr(const DecodeArgs &a, int group, hipStream_t s);

template <int D, int G>
static void launch_decode_mfma(const DecodeArgs &a, hipStream_t s) {
    const dim3 block(64 * a.heads_per_wg);
    const int64_t nwg = a.plan > 0 ? a.plan : (int64_t)a.head_groups * a.max_splits * a.num_seqs;
    const dim3 grid((unsigned)nwg);
    if (a.pool.lbs >= 4)
        hipLaunchKernelGGL((decode_mfma_kernel<D, G, true>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_mfma_kernel<D, G, false>), grid, block, 0, s, a);
}

#ifdef PKV_DECODE_ACC_VGPR

hipError_t launch_decode_mfma_vgpr(const DecodeArgs &a, int group, hipStream_t s) {
    switch (group) {
        case 1: launch_decode_mfma<128, 1>(a, s); break;
        case 2: launch_decode_mfma<128, 2>(a, s); break;
        case 4: launch_decode_mfma<128, 4>(a, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

#else

template <int DT, int D, int G>
static hipError_t run_decode(const DecodeArgs &a, hipStream_t s) {
    hipError_t e = hipSuccess;
    if constexpr (DT == 1) {
        if constexpr (kAccVgprObject<D, G>) {
            e = launch_decode_mfma_vgpr(a, G, s);
        } else {
            launch_decode_mfma<D, G>(a, s);
            e = hipGetLastError();
        }
    } else {
        const dim3 block(64 * a.heads_per_wg);
        const int64_t nwg = a.plan > 0 ? a.plan : (int64_t)a.head_groups * a.max_splits * a.num_seqs;
        hipLaunchKernelGGL((decode_valu_kernel<DT, D, G>), dim3((unsigned)nwg), block, 0, s, a);
        e = hipGetLastError();
    }
    if (e != hipSuccess || a.max_splits == 1 || a.fused_merge) return e;
    hipLaunchKernelGGL((reduce_kernel<DT, D>), dim3((unsigned)((int64_t)a.num_seqs * a.num_q_heads)),
                       dim3(kReduceThreads), (size_t)a.max_splits * sizeof(float), s, a);
    return hipGetLastError();
}

typedef hipError_t (*DecodeFn)(const DecodeArgs &, hipStream_t);

// int8 / int4 pools (QB bits per code): bf16 queries and outputs, split
// and planned schedules.
template <int D, int G, int QB>
static hipError_t run_decode_q8(const DecodeArgs &a, hipStream_t s) {
    const dim3 block(64 * a.heads_per_wg);
    const dim3 grid((unsigned)(a.plan > 0 ? a.plan : (int64_t)a.head_groups * a.max_splits * a.num_seqs));
    if (a.pool.lbs >= 4)
        hipLaunchKernelGGL((decode_q8_kernel<D, G, true, QB>), grid, block, 0, s, a);
    else
        hipLaunchKernelGGL((decode_q8_kernel<D, G, false, QB>), grid, block, 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_splits == 1 || a.fused_merge) return e;
    hipLaunchKernelGGL((reduce_kernel<1, D>), dim3((unsigned)((int64_t)a.num_seqs * a.num_q_heads)),
                       dim3(kReduceThreads), (size_t)a.max_splits * sizeof(float), s, a);
    return hipGetLastError();
}

template <int D, int QB>
static DecodeFn pick_group_q8(int group) {
    switch (group) {
        case 1: return run_decode_q8<D, 1, QB>;
        case 2: return run_decode_q8<D, 2, QB>;
        case 4: return run_decode_q8<D, 4, QB>;
        case 8: return run_decode_q8<D, 8, QB>;
        default: return nullptr;
    }
}

template <int DT, int D>
static DecodeFn pick_group(int group) {
    switch (group) {
        case 1: return run_decode<DT, D, 1>;
        case 2: return run_decode<DT, D, 2>;
        case 4: return run_decode<DT, D, 4>;
        case 8: return run_decode<DT, D, 8>;
        default: return nullptr;
    }
}

template <int DT>
static DecodeFn pick_dim(int head_dim, int group) {
    switch (head_dim) {
        case 64: return pick_group<DT, 64>(group);
        case 128: return pick_group<DT, 128>(group);
        default: return nullptr;
    }
}

static DecodeFn pick(int dtype, int head_dim, int group) {
    if (dtype == 0) return pick_dim<0>(head_dim, group);
    if (dtype == 1) return pick_dim<1>(head_dim, group);
    if (dtype == 2) {
        if (head_dim == 64) return pick_group_q8<64, 8>(group);
        if (head_dim == 128) return pick_group_q8<128, 8>(group);
    }
    if (dtype == 3) {
        if (head_dim == 64) return pick_group_q8<64, 4>(group);
        if (head_dim == 128) return pick_group_q8<128, 4>(group);
    }
    return nullptr;
}

bool decode_supported(int dtype, int head_dim, int group) {
    return pick(dtype, head_dim, group) != nullptr;
}

hipError_t launch_decode(const DecodeArgs &a, int dtype, int head_dim, int group, hipStream_t s) {
    DecodeFn f = pick(dtype, head_dim, group);
    if (!f) return hipErrorInvalidValue;
    return f(a, s);
}

#endif  // PKV_DECODE_ACC_VGPR

}  // namespace pkv
