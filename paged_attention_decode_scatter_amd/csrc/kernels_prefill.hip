// kernels_prefill.hip -- prefill / append attention over the paged pool.
//
// The last n = q_start[s+1] - q_start[s] tokens of sequence s are its
// queries; query i sits at logical position P_i = L - n + i and attends
// causally to logical tokens 0 .. P_i, read in place through the block
// table (first-block offset honoured) -- the prefill of "vLLM PagedAttention
// source notes" sec. 2.4 (the prompt's K/V written, then attended) over the
// tables of mini-runtime ch. 12 sec. 2.2, so that a request whose prefix
// blocks are shared attends to them without copies.  A query with P_i < 0
// (more queries than tokens) sees nothing and gets zeros.  n = 1 is decode.
//
// bf16 kernel (matrix cores).  Workgroup = (kv head, sequence, query
// tile), max(4, G) wavefronts; wavefront w handles query head kv*G + w % G and the
// tile's (w / G)-th group of 48 (head_dim 128) or 64 (64) queries, in sub-tiles of 16 that are
// its MFMA columns.  Keys go in stages of two 16-position chunks:
//   the workgroup loads each chunk's K rows (registers, then a padded LDS
//   tile) and V rows (straight into LDS) once for all its wavefronts, in a
//   ring of two stages, one computed while the next one's loads are in
//   flight, with one barrier per stage; for each of its sub-tiles a
//   wavefront does S^T = K . Q^T for both chunks (v_mfma_f32_16x16x32_bf16),
//   masks per element (outside the sequence, missing block, or key after
//   the query), and runs one online-softmax step per query column over the
//   32 keys (lazy reference max, exp2 domain); then O += P . V with one
//   v_mfma_f32_16x16x32_bf16 per sub-tile and 16 output columns, its V
//   operand the two chunks' transposing LDS reads side by side -- the
//   decode kernel's per-chunk step, with queries in place of heads.
// fp32 kernel (VALU): one work item per (query row, group of kv heads), the
//   decode VALU loop over the keys the query sees.
#include "attn_common.h"

namespace pkv {

namespace {

// Table entries covering flat positions [lo, hi) into bt_s (entry jb0
// first); ids outside the pool or past the table become -1.  Whole
// workgroup; ends with a barrier.
__device__ __forceinline__ int64_t stage_entries(const PrefillArgs &a, int seq, int64_t lo,
                                                 int64_t hi, int32_t *bt_s) {
    const int lbs = a.pool.lbs;
    const int64_t jb0 = lo >> lbs;
    const int nbt = hi > lo ? (int)(((hi - 1) >> lbs) - jb0 + 1) : 0;
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

}  // namespace

template <int D, int G, bool UB>
__global__ __launch_bounds__(64 * kPrefillWaves<G>) __attribute__((amdgpu_waves_per_eu(2))) void prefill_mfma_kernel(
    PrefillArgs a) {
    using S = MfmaShape<D>;
    constexpr int ROWB = S::ROWB, PPR = S::PPR, NP = S::NP, KS = S::KS, NV = S::NV;
    constexpr int VSLAB = S::VSLAB, VTILE = S::VTILE;
    constexpr int NB = kPrefillRing;            // chunks in the LDS ring (3 stages of 2)
    constexpr int KFRAG = KS * 1024;            // one chunk's K in A-operand fragment order
    constexpr int NW = kPrefillWaves<G>;        // wavefronts: G heads x NW / G query groups
    constexpr int LPW = (NP + NW - 1) / NW;     // V tile-load instructions per wave (at most)
    constexpr int KPW = (KS + NW - 1) / NW;     // K fragment copies per wave (at most)
    constexpr int QW = kPrefillWaveQueries<D, G>;   // queries per wavefront
    constexpr int QT = QW / 16;                 // 16-query sub-tiles per wavefront
    constexpr float kLazy = 8.0f;
    constexpr float kMinRef = -0x1p127f;
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    __shared__ int32_t bt_s[kBtLds];
    __shared__ __attribute__((aligned(16))) char kfrag[NB][KFRAG];
    __shared__ __attribute__((aligned(16))) char vtile[NB][VTILE];

    // (kv head, sequence, tile), tile fastest; neighbours share an XCD so
    // the tiles of one sequence reuse its K/V in one L2
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int lid = xcd * (nwg >> 3) + min(xcd, nwg & 7) + (bid >> 3);
    const int tile = lid % a.q_tiles;
    const int rest = lid / a.q_tiles;
    const int seq = rest % a.num_seqs;
    const int hk = rest / a.num_seqs;
    const int64_t row0 = a.q_start[seq];
    const int64_t n = (int64_t)a.q_start[seq + 1] - row0;
    const int qt0 = kPrefillTile<D, G> * tile;    // the workgroup's first query
    const int64_t nlim = min(n, (int64_t)a.max_q_len);   // queries computed
    if (qt0 >= nlim) return;  // uniform
    const int64_t L = a.seq_lens[seq];
    const int64_t off = a.offsets[seq];
    // last query position of the workgroup: the key range it stages
    const int64_t pmax = L - n + min((int64_t)qt0 + kPrefillTile<D, G>, nlim) - 1;

    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    const int cn = lane & 15;   // MFMA column: query q0 + 16 t + cn / output column
    const int g4 = lane >> 4;
    const int hq = hk * G + w % G;
    // this wavefront's queries: q0 .. q0 + nq - 1 (nq may be <= 0: it then
    // only helps load and takes part in the barriers)
    const int q0 = qt0 + QW * (w / G);
    const int nq = (int)max((int64_t)0, min((int64_t)QW, nlim - q0));
    const int64_t pmin = L - n + q0;            // its first query's position

    // Q^T fragments of sub-tile t: column cn = query q0 + 16 t + cn of head hq
    u32x4 qf[QT][KS];
    int qpos[QT];       // this column's query position in sub-tile t (-1: none)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        const int qi = 16 * t + cn;
        qpos[t] = qi < nq ? (int)(pmin + qi) : -1;
        const char *qp = a.q + ((row0 + q0 + qi) * a.num_q_heads + hq) * (int64_t)(D * 2) + 16 * g4;
#pragma unroll
        for (int j = 0; j < KS; ++j) qf[t][j] = qi < nq ? ld16(qp + 64 * j) : u32x4{0, 0, 0, 0};
    }
    // m_h[t]: reference max of query column cn (exp2 domain); acc[t][sl]:
    // O rows 4*g4 + i, columns 16 sl + cn; accl[t]: the denominators of the
    // same rows, accumulated on the matrix core as P . (a column of ones),
    // so they sum exactly the bf16 P values the P . V product uses and land
    // in the output rows' layout.  m_h starts at a finite value below any
    // score (kMinRef): the first live score of a column always moves it,
    // with the old contribution scaled by exp2(kMinRef - m) = 0, and masked
    // scores (-inf) still give exp2(-inf) = 0, so no -inf special case
    // remains in the loop.
    float m_h[QT];
    f32x4 acc[QT][NV], accl[QT];
#pragma unroll
    for (int t = 0; t < QT; ++t) {
        m_h[t] = kMinRef;
        accl[t] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int sl = 0; sl < NV; ++sl) acc[t][sl] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0 pairs

    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;
    const int64_t row_bytes = a.pool.row_bytes;
    const float sl2 = a.scale_log2;
    const char *kh = a.pool.k + a.pool.layer_off + (int64_t)hk * ROWB;
    const char *vh = a.pool.v + a.pool.layer_off + (int64_t)hk * ROWB;
    const int trow = lane / PPR;
    const int tpp = lane % PPR;
    // V tile swizzle (head_dim 128): a row at an odd position of its slab
    // holds its 16-byte pieces in the order piece ^ 8, so that the
    // transposed reads of lane groups g4 = 2h and 2h + 1 (rows at positions
    // 2h and 2h + 1, the same slabs) fall in opposite 128-byte halves of
    // the banks.  A copy lane fetches the piece it stores (same row bytes).
    constexpr bool kVSwz = PKV_PREFILL_VSWZ && D == 128;
    const int tsrc = kVSwz ? (tpp ^ (8 * (trow & 1))) : tpp;
    // the wavefronts share a chunk's KS + NP copy instructions round robin,
    // K fragments first: K fragment j by wave j % NW, V instruction i by
    // wave (KS + i) % NW; this wave's first V instruction:
    const int iv0 = ((w - KS) % NW + NW) % NW;

    if (pmax >= 0) {
        // Positions are 32-bit from here on (flat positions of a table stay
        // below 2^31; 64-bit arithmetic cost registers and spills here).
        const int32_t off32 = (int32_t)off, pmin32 = (int32_t)pmin;
        // keys: logical 0 .. pmax = flat [off, off + pmax + 1), staged in pieces
        const int32_t klo = off32, khi = (int32_t)(off + pmax + 1);
        for (int32_t plo = klo & ~15; plo < khi; plo += 16 * a.seg_chunks) {
            const int32_t phi = min(khi, plo + 16 * a.seg_chunks);
            const int32_t lo = max(plo, klo);
            __syncthreads();  // the previous piece's entries and tiles are done with
            const int32_t jb0 = (int32_t)stage_entries(a, seq, lo, phi, bt_s);
            const int32_t first = lo & ~15;
            const int32_t last = (phi - 1) & ~15;

            // This wave's share of a chunk's loads, all global -> LDS: K
            // fragments j = w, w + NW, .. (lane (cn, g4) copies the 16 bytes
            // of row cn it later reads as its A operand for step j, so the
            // tile is in fragment order and its reads are contiguous) and V
            // tile-load instructions i = iv0, iv0 + NW, .. (row layout).
            auto load_chunk = [&](int32_t pc, int slot) {
                char *kd = kfrag[slot];
                char *vd = vtile[slot];
                if constexpr (UB) {
                    // the chunk lies in one block: a wave-uniform base
                    const int32_t b = __builtin_amdgcn_readfirstlane(bt_s[(pc >> lbs) - jb0]);
                    const int64_t base = (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride +
                                         (int64_t)(pc & (int32_t)bsm) * row_bytes;
                    const char *kb = kh + base;
                    const char *vb = vh + base;
#pragma unroll
                    for (int k = 0; k < KPW; ++k) {
                        const int j = w + NW * k;
                        if (j < KS)
                            lds_copy16(kb + (uint32_t)(cn * (int32_t)row_bytes + 16 * g4 + 64 * j), kd + 1024 * j);
                    }
#pragma unroll
                    for (int k = 0; k < LPW; ++k) {
                        const int i = iv0 + NW * k;
                        if (i < NP)
                            lds_copy16(vb + (uint32_t)((i + NP * trow) * (int32_t)row_bytes + 16 * tsrc), vd + i * VSLAB);
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < KPW; ++k) {
                        const int j = w + NW * k;
                        if (j < KS) {
                            const int32_t p = pc + cn;
                            const bool in = p >= lo && p < phi;
                            const int32_t b = in ? bt_s[(p >> lbs) - jb0] : -1;
                            const int64_t o = (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride +
                                              (int64_t)(p & (int32_t)bsm) * row_bytes + 16 * g4 + 64 * j;
                            lds_copy16(kh + o, kd + 1024 * j);
                        }
                    }
#pragma unroll
                    for (int k = 0; k < LPW; ++k) {
                        const int i = iv0 + NW * k;
                        if (i < NP) {
                            const int32_t p = pc + i + NP * trow;
                            const bool in = p >= lo && p < phi;
                            const int32_t b = in ? bt_s[(p >> lbs) - jb0] : -1;
                            const int64_t o = (int64_t)(b >= 0 ? b : 0) * a.pool.block_stride +
                                              (int64_t)(p & (int32_t)bsm) * row_bytes + 16 * tsrc;
                            lds_copy16(vh + o, vd + i * VSLAB);
                        }
                    }
                }
            };
            // rows of chunk pc that hold a token of the sequence
            auto row_ok = [&](int32_t pc, int row) -> bool {
                const int32_t p = pc + row;
                if (p < lo || p >= phi) return false;
                return bt_s[(p >> lbs) - jb0] >= 0;
            };
            // every row of chunk pc holds a token (wave-uniform; block
            // size >= 16 only)
            auto chunk_live = [&](int32_t pc) -> bool {
                if constexpr (UB) return pc >= lo && pc + 16 <= phi && bt_s[(pc >> lbs) - jb0] >= 0;
                return false;
            };

            // Two chunks per stage and one barrier per stage: a ring of six
            // chunk slots holds three stages, one being computed while the
            // next two stages' loads are in flight.
            static_assert(NB == 6, "three stages of two chunks");
            // One softmax step over the stage's two chunks, cpc (slot qs)
            // and cpc + 16 (slot qs + 1).  Lane group g4 holds the scores of
            // rows 4*g4 .. 4*g4+3 of each chunk; P.V contracts those 8 keys
            // per lane group with one v_mfma_f32_16x16x32_bf16, whose P
            // operand (A) and V operand (B) both list the first chunk's rows
            // then the second's (the same relabelling of the 32 keys in
            // both operands, so the sum is unchanged).
            auto compute_stage = [&](int32_t cpc, int qs) {
                // the two chunks' K fragments: slot qs + 1 follows slot qs,
                // fragment j of chunk c at 1024 (KS c + j)
                static_assert(KFRAG == 1024 * KS && (KS == 4 || KS == 2), "K fragment layout");
                u32x4 kf[2][KS];
                {
                    u32x4 kr[2 * KS];
                    if constexpr (KS == 4) lds_read16_x8<1024>(kfrag[qs] + 16 * lane, kr);
                    else lds_read16_x4<1024>(kfrag[qs] + 16 * lane, kr);
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int j = 0; j < KS; ++j) kf[c][j] = kr[KS * c + j];
                }
                // A chunk needs no mask when all its rows are live tokens at
                // or before the wavefront's first query.  When both chunks are
                // such (every stage below the causal diagonal and inside the
                // piece: nearly all of them), the stage takes the unmasked
                // path (wave-uniform branch); else the rows' liveness is
                // found once for the stage and each score is masked.  A
                // stage without a second chunk re-reads the last one into
                // the second slot, whose rows then fail row_ok: masked.
                bool full[2];
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    const int32_t pcc = cpc + 16 * c;
                    full[c] = nq > 0 && pcc + 15 - off32 <= pmin32 && chunk_live(pcc);
                }
                const bool unmasked = full[0] && full[1];
                bool live[2][4];
                if (!unmasked) {
#pragma unroll
                    for (int c = 0; c < 2; ++c)
#pragma unroll
                        for (int i = 0; i < 4; ++i) live[c][i] = full[c] || row_ok(cpc + 16 * c, 4 * g4 + i);
                }
                // row i of chunk c holds the key at logical position kp0 + 16 c + i
                const int kp0 = cpc - off32 + 4 * g4;
                // S^T of every sub-tile first (independent accumulation
                // chains back to back on the matrix core): lane holds
                // S[token 16 c + 4*g4 + i][query 16 t + cn] (raw scores: the
                // scale is applied in the exponent; it is positive, so
                // maxima commute with it)
                f32x4 sacc[QT][2];
#pragma unroll
                for (int t = 0; t < QT; ++t)
#pragma unroll
                    for (int c = 0; c < 2; ++c)
                        sacc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            as_bf16x8(kf[c][0]), as_bf16x8(qf[t][0]), f32x4{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
#pragma unroll
                for (int j = 1; j < KS; ++j)
#pragma unroll
                    for (int t = 0; t < QT; ++t)
#pragma unroll
                        for (int c = 0; c < 2; ++c)
                            sacc[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kf[c][j]),
                                                                                 as_bf16x8(qf[t][j]), sacc[t][c], 0, 0, 0);
                if (!unmasked) {
#pragma unroll
                    for (int t = 0; t < QT; ++t)
#pragma unroll
                        for (int c = 0; c < 2; ++c)
#pragma unroll
                            for (int i = 0; i < 4; ++i)
                                sacc[t][c][i] =
                                    (live[c][i] && kp0 + 16 * c + i <= qpos[t]) ? sacc[t][c][i] : kNegInf;
                }
                // The reference max moves only when a column's max exceeds
                // it by more than kLazy (exp2 domain).  A column's max does
                // so exactly when one of its lanes' maxima does (the scaling
                // is monotone), so the lanes' own maxima decide, in one
                // wave-wide vote for all sub-tiles, whether the column
                // reductions are needed at all.  (maximum: the
                // NaN-propagating max, one v_maximum3_f32 per three inputs
                // without quieting them first.)
                float lm[QT];
                bool up = false;
#pragma unroll
                for (int t = 0; t < QT; ++t) {
                    const f32x4 &x = sacc[t][0], &y = sacc[t][1];
                    lm[t] = __builtin_elementwise_maximum(
                        __builtin_elementwise_maximum(
                            __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[0], x[1]), x[2]),
                            __builtin_elementwise_maximum(__builtin_elementwise_maximum(x[3], y[0]), y[1])),
                        __builtin_elementwise_maximum(y[2], y[3]));
                    up = up || lm[t] * sl2 > m_h[t] + kLazy;
                }
                if (__builtin_amdgcn_ballot_w64(up) != 0) {   // rare; wave-uniform
#pragma unroll
                    for (int t = 0; t < QT; ++t) {
                        const float cm = max_xor32(max_xor16(lm[t])) * sl2;
                        float alpha = 1.0f;
                        if (cm > m_h[t] + kLazy) {
                            alpha = fast_exp2(m_h[t] - cm);
                            m_h[t] = cm;
                        }
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float al = __shfl(alpha, 4 * g4 + i);
                            accl[t][i] *= al;
#pragma unroll
                            for (int sl = 0; sl < NV; ++sl) acc[t][sl][i] *= al;
                        }
                    }
                }
                // P = exp2(S * scale - m) in bf16 (exp2(-inf) = 0 for the
                // masked entries)
                u32x4 pa[QT];
#pragma unroll
                for (int t = 0; t < QT; ++t) {
                    uint32_t pp[4];
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        pp[k] = pack_bf16x2(fast_exp2(fmaf(sacc[t][k >> 1][2 * (k & 1)], sl2, -m_h[t])),
                                            fast_exp2(fmaf(sacc[t][k >> 1][2 * (k & 1) + 1], sl2, -m_h[t])));
                    pa[t] = u32x4{pp[0], pp[1], pp[2], pp[3]};
                }
                // V operand of slice sl: the transposed 4-row fragments of
                // both chunks, then every sub-tile
                const int vrow = 4 * g4 + (cn >> 2);
                const int vbase = (vrow % NP) * VSLAB + (vrow / NP) * ROWB + 8 * (cn & 3);
                // swizzled rows (odd positions): pieces 0..7 (slices 0..3)
                // sit 128 bytes later, pieces 8..15 128 bytes earlier
                const int vodd = kVSwz ? 128 * ((vrow / NP) & 1) : 0;
                static_assert(NV % 4 == 0, "V slices in groups of four");
#pragma unroll
                for (int sg = 0; sg < NV / 4; ++sg) {
                    // slices 4 sg .. 4 sg + 3 of both chunks (slot qs + 1
                    // follows slot qs)
                    uint64_t vr[8];
                    lds_read_tr16_x8<32, VTILE>(vtile[qs] + vbase + 128 * sg + (4 * sg < NV / 2 ? vodd : -vodd), vr);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const u32x4 vb = {(uint32_t)vr[k], (uint32_t)(vr[k] >> 32), (uint32_t)vr[4 + k],
                                          (uint32_t)(vr[4 + k] >> 32)};
#pragma unroll
                        for (int t = 0; t < QT; ++t)
                            acc[t][4 * sg + k] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                as_bf16x8(pa[t]), as_bf16x8(vb), acc[t][4 * sg + k], 0, 0, 0);
                    }
                }
#pragma unroll
                for (int t = 0; t < QT; ++t)
                    accl[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(pa[t]), as_bf16x8(ones), accl[t], 0, 0, 0);
            };
            // the loads of stage st (chunks first + 32 st, + 16; a second
            // chunk past the last re-reads it, masked in compute_stage)
            const int nst = ((last - first) >> 5) + 1;
            auto issue = [&](int st, int slot0) {
                const int32_t pc = first + 32 * st;
                load_chunk(pc, slot0);
                load_chunk(min(pc + 16, last), slot0 + 1);
            };
            // this wave's vector-memory operations per stage (wave-uniform)
            const int ops = 2 * ((KS + NW - 1 - w) / NW + (NP + NW - 1 - iv0) / NW);
            auto wait_stage = [&](bool next_in_flight) {
                const int n = next_in_flight ? ops : 0;
                // the copy engine's LDS writes are not tracked by the
                // compiler: an explicit wait, immediate per case
                if (n >= 8) __builtin_amdgcn_s_waitcnt(8 | (0x7 << 4) | (0xF << 8));
                else if (n >= 4) __builtin_amdgcn_s_waitcnt(4 | (0x7 << 4) | (0xF << 8));
                else if (n >= 2) __builtin_amdgcn_s_waitcnt(2 | (0x7 << 4) | (0xF << 8));
                else __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
            };
            issue(0, 0);
            if (nst > 1) issue(1, 2);
            // one loop body (no unrolling over the ring: the copies' register
            // allocations differed and moved registers between them); r is
            // stage st's ring position (slots 2r, 2r + 1), wave-uniform
            int r = 0;
            for (int st = 0; st < nst; ++st) {
                const int32_t pc = first + 32 * st;
                wait_stage(st + 1 < nst);   // this stage's loads have landed
                wave_lds_order();
                // zero the V rows of this wave's pieces that hold no live token
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                    if (!chunk_live(pc + 16 * c)) {
#pragma unroll
                        for (int k = 0; k < LPW; ++k) {
                            const int i = iv0 + NW * k;
                            if (i < NP && !row_ok(pc + 16 * c, i + NP * trow))
                                *reinterpret_cast<u32x4 *>(vtile[2 * r + c] + i * VSLAB + 16 * lane) =
                                    u32x4{0, 0, 0, 0};
                        }
                    }
                }
                __syncthreads();  // the stage's tiles complete; stage st - 1's slots free
                if (st + 2 < nst) issue(st + 2, r == 0 ? 4 : 2 * r - 2);
                compute_stage(pc, 2 * r);
                r = r == 2 ? 0 : r + 1;
            }
            // drain the copies before the tiles are restaged or released
            __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xF << 8));
        }
    }

    // out[row, hq, :] = acc / l for the tile's queries (sub-tile t, rows 4*g4 + i)
#pragma unroll
    for (int t = 0; t < QT; ++t) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int qi = 16 * t + 4 * g4 + i;
            const float lq = accl[t][i];
            if (qi < nq) {
                // one reciprocal per row and the hardware's nearest-even
                // conversion (a division and a software rounding per element
                // were a sixth of the kernel's VALU instructions)
                const float rl = lq > 0.0f ? __builtin_amdgcn_rcpf(lq) : 0.0f;
                uint16_t *o = reinterpret_cast<uint16_t *>(a.out) + ((row0 + q0 + qi) * a.num_q_heads + hq) * D + cn;
#pragma unroll
                for (int sl = 0; sl < NV; ++sl) o[16 * sl] = (uint16_t)pack_bf16x2(acc[t][sl][i] * rl, 0.0f);
            }
        }
    }
}

// fp32 pools: one workgroup per (query row, group of heads_per_wg kv heads);
// wavefront = one kv head with its G query heads, the decode VALU loop over
// the keys the query sees.
template <int DT, int D, int G>
__global__ __launch_bounds__(256) void prefill_valu_kernel(PrefillArgs a) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int VEC = 16 / E;
    constexpr int LPR = D / VEC;
    constexpr int RPI = 64 / LPR;
    constexpr int NP = kChunkTokens / RPI;
    static_assert(LPR >= 4 && LPR <= 64 && RPI <= kChunkTokens, "head_dim out of range");
    __shared__ int32_t bt_s[kBtLds];

    const int64_t row = blockIdx.x / a.head_groups;
    const int hg = blockIdx.x - (int)(row * a.head_groups);
    // the sequence of this row: q_start[seq] <= row < q_start[seq + 1]
    int lo = 0, hi = a.num_seqs;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (a.q_start[mid] <= row) lo = mid;
        else hi = mid;
    }
    const int seq = lo;
    const int64_t n = (int64_t)a.q_start[seq + 1] - a.q_start[seq];
    const int64_t qi = row - a.q_start[seq];
    if (qi >= a.max_q_len) return;  // uniform: queries past max_q_len are not computed
    const int64_t L = a.seq_lens[seq];
    const int64_t off = a.offsets[seq];
    const int64_t P = L - n + qi;

    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = hg * a.heads_per_wg + w;
    const int r = lane / LPR;
    const int c = lane % LPR;
    const int hq0 = h * G;
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;

    float m[G], l[G], acc[G][VEC];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        m[g] = kNegInf;
        l[g] = 0.0f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = 0.0f;
    }
    u32x4 qv[G];
    {
        const char *qp = a.q + (row * a.num_q_heads + hq0) * (int64_t)(D * E) + c * 16;
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g] = ld16(qp + g * (D * E));
    }
    const char *kb = a.pool.k + a.pool.layer_off + (int64_t)h * (D * E) + c * 16;
    const char *vb = a.pool.v + a.pool.layer_off + (int64_t)h * (D * E) + c * 16;

    const int64_t klo = off, khi = P >= 0 ? off + P + 1 : off;
    for (int64_t plo = klo; plo < khi; plo += 16ll * a.seg_chunks) {
        const int64_t phi = min(khi, plo + 16ll * a.seg_chunks);
        __syncthreads();
        const int64_t jb0 = stage_entries(a, seq, plo, phi, bt_s);
        for (int64_t pc = plo; pc < phi; pc += kChunkTokens) {
            u32x4 kx[NP], vx[NP];
            bool ok[NP];
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const int64_t p = pc + i * RPI + r;
                ok[i] = false;
                kx[i] = u32x4{0, 0, 0, 0};
                vx[i] = u32x4{0, 0, 0, 0};
                if (p < phi) {
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
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float cm = s[0][g];
#pragma unroll
                for (int i = 1; i < NP; ++i) cm = fmaxf(cm, s[i][g]);
                cm = cross_rows_max<LPR>(cm);
                const float mn = fmaxf(m[g], cm);
                const float alpha = mn == kNegInf ? 1.0f : fast_exp2(m[g] - mn);
                float ps = 0.0f;
                float p[NP];
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    p[i] = s[i][g] == kNegInf ? 0.0f : fast_exp2(s[i][g] - mn);
                    ps += p[i];
                }
                l[g] = fmaf(l[g], alpha, ps);
#pragma unroll
                for (int e = 0; e < VEC; ++e) acc[g][e] *= alpha;
                m[g] = mn;
#pragma unroll
                for (int i = 0; i < NP; ++i) {
                    float vf[VEC];
                    unpack16<DT>(vx[i], vf);
#pragma unroll
                    for (int e = 0; e < VEC; ++e) acc[g][e] = fmaf(p[i], vf[e], acc[g][e]);
                }
            }
        }
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        l[g] = cross_rows_sum<LPR>(l[g]);
#pragma unroll
        for (int e = 0; e < VEC; ++e) acc[g][e] = cross_rows_sum<LPR>(acc[g][e]);
    }
    if (r != 0) return;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float o[VEC];
#pragma unroll
        for (int e = 0; e < VEC; ++e) o[e] = l[g] > 0.0f ? acc[g][e] / l[g] : 0.0f;
        store16<DT>(a.out + ((row * a.num_q_heads + hq0 + g) * D + c * VEC) * E, o);
    }
}

namespace {

template <int DT, int D, int G>
hipError_t run_prefill(const PrefillArgs &a, hipStream_t s) {
    if constexpr (DT == 1) {
        const int64_t nwg = (int64_t)a.q_tiles * a.num_seqs * a.num_kv_heads;
        if (a.pool.lbs >= 4)
            hipLaunchKernelGGL((prefill_mfma_kernel<D, G, true>), dim3((unsigned)nwg), dim3(64 * kPrefillWaves<G>), 0, s, a);
        else
            hipLaunchKernelGGL((prefill_mfma_kernel<D, G, false>), dim3((unsigned)nwg), dim3(64 * kPrefillWaves<G>), 0, s, a);
    } else {
        const int64_t nwg = (int64_t)a.num_q_rows * a.head_groups;
        hipLaunchKernelGGL((prefill_valu_kernel<DT, D, G>), dim3((unsigned)nwg), dim3(64 * a.heads_per_wg), 0, s,
                           a);
    }
    return hipGetLastError();
}

typedef hipError_t (*PrefillFn)(const PrefillArgs &, hipStream_t);

template <int DT, int D>
PrefillFn pick_group(int group) {
    switch (group) {
        case 1: return run_prefill<DT, D, 1>;
        case 2: return run_prefill<DT, D, 2>;
        case 4: return run_prefill<DT, D, 4>;
        case 8: return run_prefill<DT, D, 8>;
        default: return nullptr;
    }
}

PrefillFn pick(int dtype, int head_dim, int group) {
    if (dtype != 0 && dtype != 1) return nullptr;
    if (head_dim == 64) return dtype ? pick_group<1, 64>(group) : pick_group<0, 64>(group);
    if (head_dim == 128) return dtype ? pick_group<1, 128>(group) : pick_group<0, 128>(group);
    return nullptr;
}

}  // namespace

bool prefill_supported(int dtype, int head_dim, int group) { return pick(dtype, head_dim, group) != nullptr; }

hipError_t launch_prefill(const PrefillArgs &a, int dtype, int head_dim, int group, hipStream_t s) {
    PrefillFn f = pick(dtype, head_dim, group);
    if (!f) return hipErrorInvalidValue;
    return f(a, s);
}

}  // namespace pkv
