// kernels_copy.hip -- integer-index kernels for gfx950: slot computation,
// slot_mapping scatter, block_table gather, whole-block copies, contract
// validation.
//
// Sources:
//   [P1] mini-vllm tutorial, "step14_2 - index_select gather"
//   [P2] "vLLM PagedAttention source notes"
//   [P3] mini-runtime, chapter 12 "Paged KV Cache"
//
// Scatter and gather are pure byte moves: every lane moves whole 16-byte
// pieces of a row (global_load/store_dwordx4), consecutive lanes cover
// consecutive pieces of a row, so each wavefront instruction touches full
// 128-byte lines.  Several pieces are loaded before any is stored to keep
// enough bytes in flight per CU for HBM.
#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 ld16(const char *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}
__device__ __forceinline__ u32x4 ld16_stream(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}
__device__ __forceinline__ void st16(char *p, u32x4 v) {
    *reinterpret_cast<u32x4 *>(p) = v;
}
__device__ __forceinline__ void st16_stream(char *p, u32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<u32x4 *>(p));
}

// Unroll depth of the copy loops (16-byte pieces per tensor in flight per
// lane before the first store).  With 8 and the streaming (nontemporal)
// hints -- on the scattered pool stores and on the gather's pool loads,
// bytes no later access of the same call reuses -- the prefill-shape
// scatter and gather went from 13.7 / 15.4 us to 11.3 / 12.3 us on MI355X.
constexpr int kUnroll = 8;

// ---------------------------------------------------------------------------
// Slot of each new token: table[seq][(off+pos) >> lbs] << lbs | (off+pos) & bsm
// [P2 sec. 2.2 slot formula; P3 sec. 2.2 first-block offset].
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void slot_mapping_kernel(SlotArgs a) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= a.num_tokens) return;
    const int32_t seq = a.token_seq[i];
    int64_t slot = -1;
    if (seq >= 0 && seq < a.num_seqs) {
        const int64_t pos = a.token_pos[i];
        const int64_t p = (int64_t)a.offsets[seq] + pos;
        const int64_t j = p >> a.lbs;
        if (pos >= 0 && p >= 0 && j < a.bt_stride) {
            const int32_t b = a.block_tables[(int64_t)seq * a.bt_stride + j];
            if (b >= 0) slot = ((int64_t)b << a.lbs) | (p & ((1 << a.lbs) - 1));
        }
    }
    a.slots[i] = slot;
}

hipError_t launch_slot_mapping(const SlotArgs &a, hipStream_t s) {
    const int64_t blocks = (a.num_tokens + 255) / 256;
    hipLaunchKernelGGL(slot_mapping_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Scatter [P1 "relation to step14_1"; P2 sec. 2.2]: row i of k_src/v_src ->
// pool row (slot >> lbs, layer, slot & bsm).  A workgroup moves tok_per_wg
// consecutive rows; piece idx of the workgroup is (row idx / cpr, piece
// idx % cpr) so a wavefront's lanes cover consecutive pieces of a row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void scatter_kernel(ScatterArgs a) {
    const int64_t tok0 = (int64_t)blockIdx.x * a.tok_per_wg;
    const int64_t left = a.num_tokens - tok0;
    const int ntok = left < a.tok_per_wg ? (int)left : a.tok_per_wg;
    const int cpr = a.row_bytes >> 4;
    const int n = ntok * cpr;
    const int64_t bsm = (1ll << a.lbs) - 1;
    const bool has_v = a.v_src != nullptr;
    for (int base = threadIdx.x; base < n; base += kCopyThreads * kUnroll) {
        u32x4 kk[kUnroll], vv[kUnroll];
        int64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kCopyThreads;
            dst[u] = -1;
            if (idx < n) {
                int tt, ch;
                if (a.lcpr >= 0) {
                    tt = idx >> a.lcpr;
                    ch = idx & (cpr - 1);
                } else {
                    tt = idx / cpr;
                    ch = idx - tt * cpr;
                }
                const int64_t t = tok0 + tt;
                // the row is loaded with its slot, not after it (one memory
                // round trip instead of two); padding rows are read and
                // dropped
                const int64_t slot = a.slots[t];
                const int64_t src = t * a.row_bytes + ((int64_t)ch << 4);
                kk[u] = ld16_stream(a.k_src + src);
                if (has_v) vv[u] = ld16_stream(a.v_src + src);
                if (slot >= 0 && slot < a.total_slots)
                    dst[u] = (slot >> a.lbs) * a.block_stride + a.layer_off +
                             (slot & bsm) * a.row_bytes + ((int64_t)ch << 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (dst[u] >= 0) {
                st16_stream(a.kpool + dst[u], kk[u]);
                if (has_v) st16_stream(a.vpool + dst[u], vv[u]);
            }
        }
    }
}

hipError_t launch_scatter(const ScatterArgs &a, hipStream_t s) {
    const int64_t blocks = (a.num_tokens + a.tok_per_wg - 1) / a.tok_per_wg;
    hipLaunchKernelGGL(scatter_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Append: the slot computation of slot_mapping_kernel and the scatter of
// scatter_kernel for one row per token, in one kernel.  The source pieces
// are loaded while the slot is still being looked up (they depend only on
// the row), so the chain to the store is the token's sequence and position,
// its offset, its table entry.  The lane holding piece 0 of a row writes
// the slot when slots_out is given.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void append_kernel(AppendArgs a) {
    const ScatterArgs &c = a.sc;
    const int64_t tok0 = (int64_t)blockIdx.x * c.tok_per_wg;
    const int64_t left = c.num_tokens - tok0;
    const int ntok = left < c.tok_per_wg ? (int)left : c.tok_per_wg;
    const int cpr = c.row_bytes >> 4;
    const int n = ntok * cpr;
    const int64_t bsm = (1ll << c.lbs) - 1;
    const bool has_v = c.v_src != nullptr;
    for (int base = threadIdx.x; base < n; base += kCopyThreads * kUnroll) {
        u32x4 kk[kUnroll], vv[kUnroll];
        int64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kCopyThreads;
            dst[u] = -1;
            if (idx < n) {
                int tt, ch;
                if (c.lcpr >= 0) {
                    tt = idx >> c.lcpr;
                    ch = idx & (cpr - 1);
                } else {
                    tt = idx / cpr;
                    ch = idx - tt * cpr;
                }
                const int64_t t = tok0 + tt;
                const int64_t src = t * c.row_bytes + ((int64_t)ch << 4);
                kk[u] = ld16_stream(c.k_src + src);
                if (has_v) vv[u] = ld16_stream(c.v_src + src);
                const int32_t seq = a.token_seq[t];
                int64_t slot = -1;
                if (seq >= 0 && seq < a.num_seqs) {
                    const int64_t pos = a.token_pos[t];
                    const int64_t p = (int64_t)a.offsets[seq] + pos;
                    const int64_t j = p >> c.lbs;
                    if (pos >= 0 && p >= 0 && j < a.bt_stride) {
                        const int32_t b = a.block_tables[(int64_t)seq * a.bt_stride + j];
                        if (b >= 0) slot = ((int64_t)b << c.lbs) | (p & bsm);
                    }
                }
                if (ch == 0 && a.slots_out) a.slots_out[t] = slot;
                if (slot >= 0 && slot < c.total_slots)
                    dst[u] = (slot >> c.lbs) * c.block_stride + c.layer_off + (slot & bsm) * c.row_bytes +
                             ((int64_t)ch << 4);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (dst[u] >= 0) {
                st16_stream(c.kpool + dst[u], kk[u]);
                if (has_v) st16_stream(c.vpool + dst[u], vv[u]);
            }
        }
    }
}

hipError_t launch_append(const AppendArgs &a, hipStream_t s) {
    const int64_t blocks = (a.sc.num_tokens + a.sc.tok_per_wg - 1) / a.sc.tok_per_wg;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Gather [P1 "Problem"/"Solution"; P3 sec. 2.2]: out row (row_start + t) <-
// pool row (table[(off+t) >> lbs], layer, (off+t) & bsm) for t < seq_len.
// Workgroup (seq, tile) covers tokens [tile*T, tile*T + T); the table
// entries that range touches are staged in LDS first.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void gather_kernel(GatherArgs a) {
    __shared__ int32_t bt_s[kBtLds];
    const int seq = blockIdx.x / a.tiles_per_seq;
    const int tile = blockIdx.x - seq * a.tiles_per_seq;
    const int t0 = tile * a.tok_per_wg;
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;
    // The table entries this tile can touch for any offset in [0, bs) are
    // staged together with the length and offset (one memory round trip
    // instead of two): entries t0 / bs .. (t0 + tok_per_wg - 1 + bs - 1) / bs.
    // An offset outside [0, bs) breaks the contract and is clamped into it.
    const int64_t jb0 = (int64_t)t0 >> lbs;
    const int nbt = (int)((((int64_t)t0 + a.tok_per_wg - 1 + bsm) >> lbs) - jb0 + 1);
    const int L = a.seq_lens[seq];
    int64_t off = a.offsets[seq];
    for (int i = threadIdx.x; i < nbt; i += kCopyThreads) {
        const int64_t j = jb0 + i;
        int32_t b = -1;
        if (j < a.bt_stride) {
            b = a.block_tables[(int64_t)seq * a.bt_stride + j];
            if (b < 0 || b >= a.pool.num_blocks) b = -1;
        }
        bt_s[i] = b;
    }
    if (t0 >= L) return;  // uniform across the workgroup (no barrier passed yet)
    off = off < 0 ? 0 : (off > bsm ? bsm : off);
    const int t1 = min(L, t0 + a.tok_per_wg);
    __syncthreads();

    const int cpr = a.pool.row_bytes >> 4;
    const int n = (t1 - t0) * cpr;
    const int64_t row0 = a.out_row_start[seq];
    const bool has_v = a.v_out != nullptr;
    for (int base = threadIdx.x; base < n; base += kCopyThreads * kUnroll) {
        u32x4 kk[kUnroll], vv[kUnroll];
        int64_t dst[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int idx = base + u * kCopyThreads;
            dst[u] = -1;
            kk[u] = u32x4{0, 0, 0, 0};
            vv[u] = u32x4{0, 0, 0, 0};
            if (idx < n) {
                int tt, ch;
                if (a.lcpr >= 0) {
                    tt = idx >> a.lcpr;
                    ch = idx & (cpr - 1);
                } else {
                    tt = idx / cpr;
                    ch = idx - tt * cpr;
                }
                const int t = t0 + tt;
                const int64_t p = off + t;
                const int64_t orow = row0 + t;
                if (orow < 0 || orow >= a.out_rows) continue;
                dst[u] = orow * a.pool.row_bytes + ((int64_t)ch << 4);
                const int32_t b = bt_s[(int)((p >> lbs) - jb0)];
                if (b >= 0) {
                    const int64_t src = (int64_t)b * a.pool.block_stride + a.pool.layer_off +
                                        (int64_t)(p & bsm) * a.pool.row_bytes + ((int64_t)ch << 4);
                    kk[u] = ld16_stream(a.pool.k + src);
                    if (has_v) vv[u] = ld16_stream(a.pool.v + src);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (dst[u] >= 0) {
                // streaming stores: the call does not read its output back
                st16_stream(a.k_out + dst[u], kk[u]);
                if (has_v) st16_stream(a.v_out + dst[u], vv[u]);
            }
        }
    }
}

hipError_t launch_gather(const GatherArgs &a, hipStream_t s) {
    const int64_t blocks = (int64_t)a.num_seqs * a.tiles_per_seq;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Quantised pools [P3 sec. 6 names quantised KV, int8 / int4; the reading:
// one float32 scale s = max|x| / Q per (token, kv head) row, codes
// round-half-even(x / s) clamped to [-Q, Q], all in IEEE float32; Q = 127
// for int8, 7 for int4, whose codes are packed two per byte, element 2i of
// a row in the low nibble of byte i, four-bit two's complement].
//
// Quantising scatter / append: LPH = D/8 lanes hold one (token, head) row,
// 8 bf16 values each; the row's max |x| is reduced over those lanes, and
// each lane stores its 8 codes (8 bytes, or 4 for int4); the lane with
// piece 0 stores the scale.  The slot is given (kv_scatter) or computed as
// the append does.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <int Q>
__device__ __forceinline__ uint32_t quant_code(float x, float s) {
    const float c = s > 0.0f ? fminf(fmaxf(__builtin_rintf(__fdiv_rn(x, s)), -(float)Q), (float)Q) : 0.0f;
    return (uint32_t)(int32_t)c & 0xffu;
}

// 8 bf16 values (one 16-byte piece) -> 8 int8 codes (two words).
__device__ __forceinline__ uint2 quant_piece(u32x4 x, float s) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t c[2] = {0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = quant_code<127>(bf16_to_f32(w[i] & 0xffffu), s);
        const uint32_t hi = quant_code<127>(bf16_to_f32(w[i] >> 16), s);
        c[i >> 1] |= (lo | (hi << 8)) << (16 * (i & 1));
    }
    return make_uint2(c[0], c[1]);
}

// 8 bf16 values -> 8 int4 codes (one word): byte i holds element 2i in its
// low nibble and element 2i + 1 in its high nibble.
__device__ __forceinline__ uint32_t quant_piece4(u32x4 x, float s) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    uint32_t c = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t lo = quant_code<7>(bf16_to_f32(w[i] & 0xffffu), s) & 0xfu;
        const uint32_t hi = quant_code<7>(bf16_to_f32(w[i] >> 16), s) & 0xfu;
        c |= (lo | (hi << 4)) << (8 * i);
    }
    return c;
}

__device__ __forceinline__ float piece_amax(u32x4 x) {
    const uint32_t w[4] = {x.x, x.y, x.z, x.w};
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        m = fmaxf(m, fmaxf(fabsf(bf16_to_f32(w[i] & 0xffffu)), fabsf(bf16_to_f32(w[i] >> 16))));
    return m;
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// max over each aligned group of W lanes (W = 8 or 16), in every lane of the
// group: DPP within the 16-lane rows (quad swaps, then the half-row and row
// mirrors), no LDS permute round trips
template <int W>
__device__ __forceinline__ float group_max(float x) {
    static_assert(W == 8 || W == 16, "group");
    x = fmaxf(x, dpp_f<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp_f<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp_f<0x141>(x));  // row_half_mirror
    if constexpr (W == 16) x = fmaxf(x, dpp_f<0x140>(x));  // row_mirror
    return x;
}

template <int D, int QB>
__global__ __launch_bounds__(256) void scatter_q8_kernel(ScatterQ8Args a) {
    constexpr int Q = QB == 8 ? 127 : 7;
    constexpr int HB = D * QB / 8;   // bytes of one (token, head) row of codes
    constexpr int LPH = D / 8;       // lanes per (token, head) row
    constexpr int RPW = 256 / LPH;   // rows per workgroup
    const int p = threadIdx.x % LPH;
    const int64_t H = a.num_kv_heads;
    const int64_t i = (int64_t)blockIdx.x * RPW + threadIdx.x / LPH;
    const bool live = i < a.num_tokens * H;
    const int64_t tok = live ? i / H : 0;
    const int64_t h = live ? i - tok * H : 0;
    const int64_t bsm = (1ll << a.lbs) - 1;
    int64_t slot = -1;
    if (live) {
        if (a.slots) {
            slot = a.slots[tok];
        } else if (a.step_lens) {
            const int64_t L = a.step_lens[tok];
            const int64_t off = a.offsets[tok];
            if (L >= 1 && L <= a.step_max_len && off >= 0 && off <= bsm) {
                const int64_t q = off + L - 1;
                const int64_t j = q >> a.lbs;
                if (j < a.bt_stride) {
                    const int32_t b = a.block_tables[tok * a.bt_stride + j];
                    if (b >= 0) slot = ((int64_t)b << a.lbs) | (q & bsm);
                }
            }
        } else {
            const int32_t seq = a.token_seq[tok];
            if (seq >= 0 && seq < a.num_seqs) {
                const int64_t pos = a.token_pos[tok];
                const int64_t q = (int64_t)a.offsets[seq] + pos;
                const int64_t j = q >> a.lbs;
                if (pos >= 0 && q >= 0 && j < a.bt_stride) {
                    const int32_t b = a.block_tables[(int64_t)seq * a.bt_stride + j];
                    if (b >= 0) slot = ((int64_t)b << a.lbs) | (q & bsm);
                }
            }
            if (h == 0 && p == 0 && a.slots_out) a.slots_out[tok] = slot;
        }
    }
    const bool ok = slot >= 0 && slot < a.total_slots;
    const bool has_v = a.v_src != nullptr;
    const int64_t src = (tok * H + h) * (int64_t)(2 * D) + 16 * p;
    u32x4 kx = {0, 0, 0, 0}, vx = {0, 0, 0, 0};
    if (ok) {
        kx = ld16_stream(a.k_src + src);
        if (has_v) vx = ld16_stream(a.v_src + src);
    }
    // every lane takes part in the reductions (rows are LPH-lane aligned)
    const float km = group_max<LPH>(piece_amax(kx)), vm = group_max<LPH>(piece_amax(vx));
    if (!ok) return;
    const float ks = __fdiv_rn(km, (float)Q), vs = __fdiv_rn(vm, (float)Q);
    const int64_t b = slot >> a.lbs, r = slot & bsm;
    const int64_t dst = b * a.block_stride + a.layer_off + r * (H * HB) + h * HB + (QB * p);
    if constexpr (QB == 8) {
        *reinterpret_cast<uint2 *>(a.kpool + dst) = quant_piece(kx, ks);
        if (has_v) *reinterpret_cast<uint2 *>(a.vpool + dst) = quant_piece(vx, vs);
    } else {
        *reinterpret_cast<uint32_t *>(a.kpool + dst) = quant_piece4(kx, ks);
        if (has_v) *reinterpret_cast<uint32_t *>(a.vpool + dst) = quant_piece4(vx, vs);
    }
    if (p == 0) {
        const int64_t so = b * a.sc_block + (h << a.lbs) + r;
        a.ks[so] = ks;
        if (has_v) a.vs[so] = vs;
    }
}

hipError_t launch_scatter_q8(const ScatterQ8Args &a, hipStream_t s) {
    const int64_t rows = a.num_tokens * a.num_kv_heads;
    const int64_t rpw = 256 / (a.head_dim / 8);
    const dim3 grid((unsigned)((rows + rpw - 1) / rpw));
    if (a.head_dim == 128 && a.qbits == 8)
        hipLaunchKernelGGL((scatter_q8_kernel<128, 8>), grid, dim3(256), 0, s, a);
    else if (a.head_dim == 64 && a.qbits == 8)
        hipLaunchKernelGGL((scatter_q8_kernel<64, 8>), grid, dim3(256), 0, s, a);
    else if (a.head_dim == 128 && a.qbits == 4)
        hipLaunchKernelGGL((scatter_q8_kernel<128, 4>), grid, dim3(256), 0, s, a);
    else if (a.head_dim == 64 && a.qbits == 4)
        hipLaunchKernelGGL((scatter_q8_kernel<64, 4>), grid, dim3(256), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// Dequantising gather: each lane turns one 16-byte piece of a row (16 int8
// codes or 32 int4 codes) into bf16 values bf16(code * scale) (float32
// product, nearest-even).  Tokens whose table entry is missing or out of
// range give zero rows.
__device__ __forceinline__ uint32_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <int D, int QB>
__global__ __launch_bounds__(kCopyThreads) void gather_q8_kernel(GatherArgs a) {
    constexpr int CPP = 128 / QB;   // codes per 16-byte piece
    const int seq = blockIdx.x / a.tiles_per_seq;
    const int tile = blockIdx.x - seq * a.tiles_per_seq;
    const int64_t len = a.seq_lens[seq];
    const int64_t t0 = (int64_t)tile * a.tok_per_wg;
    if (t0 >= len) return;
    const int64_t left = len - t0;
    const int ntok = left < a.tok_per_wg ? (int)left : a.tok_per_wg;
    const int cpr = a.pool.row_bytes >> 4;  // 16-code pieces per row
    const int64_t off = a.offsets[seq];
    const int64_t row0 = a.out_row_start[seq];
    const int64_t bsm = (1ll << a.pool.lbs) - 1;
    const bool has_v = a.v_out != nullptr;
    for (int idx = threadIdx.x; idx < ntok * cpr; idx += kCopyThreads) {
        const int tt = idx / cpr;
        const int ch = idx - tt * cpr;
        const int64_t t = t0 + tt;
        const int64_t orow = row0 + t;
        if (orow < 0 || orow >= a.out_rows) continue;
        const int64_t p = off + t;
        const int64_t j = p >> a.pool.lbs;
        const int32_t b = j < a.bt_stride ? a.block_tables[(int64_t)seq * a.bt_stride + j] : -1;
        const bool okb = b >= 0 && b < a.pool.num_blocks;
        const int64_t h = (CPP * ch) / D;
        u32x4 o[2][CPP / 8] = {};
        for (int tsr = 0; tsr < (has_v ? 2 : 1); ++tsr) {
            if (!okb) break;
            const char *pool = tsr ? a.pool.v : a.pool.k;
            const float *sc = tsr ? a.pool.vs : a.pool.ks;
            const u32x4 c = ld16_stream(pool + (int64_t)b * a.pool.block_stride + a.pool.layer_off +
                                 (p & bsm) * a.pool.row_bytes + 16 * ch);
            const float s = sc[(int64_t)b * a.pool.sc_block + (h << a.pool.lbs) + (p & bsm)];
            const uint32_t w[4] = {c.x, c.y, c.z, c.w};
            uint32_t r[CPP / 2];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if constexpr (QB == 8) {
#pragma unroll
                    for (int k = 0; k < 2; ++k) {
                        const float lo = (float)(int8_t)(w[i] >> (16 * k)) * s;
                        const float hi = (float)(int8_t)(w[i] >> (16 * k + 8)) * s;
                        r[2 * i + k] = bf16_rne(lo) | (bf16_rne(hi) << 16);
                    }
                } else {
                    // byte k of the word: elements 2k (low nibble) and 2k + 1
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float lo = (float)((int32_t)(w[i] << (28 - 8 * k)) >> 28) * s;
                        const float hi = (float)((int32_t)(w[i] << (24 - 8 * k)) >> 28) * s;
                        r[4 * i + k] = bf16_rne(lo) | (bf16_rne(hi) << 16);
                    }
                }
            }
#pragma unroll
            for (int k = 0; k < CPP / 8; ++k) o[tsr][k] = u32x4{r[4 * k], r[4 * k + 1], r[4 * k + 2], r[4 * k + 3]};
        }
        const int64_t dst = (orow * (int64_t)cpr + ch) * (2 * CPP);
#pragma unroll
        for (int k = 0; k < CPP / 8; ++k) st16(a.k_out + dst + 16 * k, o[0][k]);
        if (has_v) {
#pragma unroll
            for (int k = 0; k < CPP / 8; ++k) st16(a.v_out + dst + 16 * k, o[1][k]);
        }
    }
}

hipError_t launch_gather_q8(const GatherArgs &a, int head_dim, int qbits, hipStream_t s) {
    const dim3 grid((unsigned)((int64_t)a.num_seqs * a.tiles_per_seq));
    if (head_dim == 128 && qbits == 8)
        hipLaunchKernelGGL((gather_q8_kernel<128, 8>), grid, dim3(kCopyThreads), 0, s, a);
    else if (head_dim == 64 && qbits == 8)
        hipLaunchKernelGGL((gather_q8_kernel<64, 8>), grid, dim3(kCopyThreads), 0, s, a);
    else if (head_dim == 128 && qbits == 4)
        hipLaunchKernelGGL((gather_q8_kernel<128, 4>), grid, dim3(kCopyThreads), 0, s, a);
    else if (head_dim == 64 && qbits == 4)
        hipLaunchKernelGGL((gather_q8_kernel<64, 4>), grid, dim3(kCopyThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Whole-block copies of copy-on-write [P3 sec. 3.1]: workgroup w copies
// piece w % pieces (kCopyBlockPiece bytes) of every layer's K and V of pair
// w / pieces.  Block contents are contiguous per tensor (all layers of a
// block follow one another), so a piece is one contiguous byte range.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void copy_blocks_kernel(CopyBlocksArgs a) {
    const int64_t pair = blockIdx.x / a.pieces;
    const int64_t piece = blockIdx.x - pair * a.pieces;
    const int32_t sb = a.src[pair];
    const int32_t db = a.dst[pair];
    if (sb < 0 || sb >= a.num_blocks || db < 0 || db >= a.num_blocks || sb == db) return;
    const int64_t start = piece * kCopyBlockPiece;
    int64_t len = a.block_bytes - start;
    if (len > kCopyBlockPiece) len = kCopyBlockPiece;
    const int n = (int)(len >> 4);
    const int64_t so = (int64_t)sb * a.block_stride + start;
    const int64_t dof = (int64_t)db * a.block_stride + start;
    const bool has_v = a.v != nullptr;
    for (int base = threadIdx.x; base < n; base += kCopyThreads * kUnroll) {
        u32x4 kk[kUnroll], vv[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = base + u * kCopyThreads;
            if (i < n) {
                kk[u] = ld16_stream(a.k + so + 16 * (int64_t)i);
                if (has_v) vv[u] = ld16_stream(a.v + so + 16 * (int64_t)i);
            }
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int i = base + u * kCopyThreads;
            if (i < n) {
                st16_stream(a.k + dof + 16 * (int64_t)i, kk[u]);
                if (has_v) st16_stream(a.v + dof + 16 * (int64_t)i, vv[u]);
            }
        }
    }
}

hipError_t launch_copy_blocks(const CopyBlocksArgs &a, hipStream_t s) {
    const int64_t blocks = a.num_pairs * a.pieces;
    hipLaunchKernelGGL(copy_blocks_kernel, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Read-rate reference (kv_read_blocks): workgroup i reads the layer slice
// of K and of V of block ids[i] (block_size rows, contiguous) with 16-byte
// loads, kUnroll per tensor in flight per lane, and writes the XOR of all
// their 32-bit words -- a value that depends on every byte, so no load can
// be dropped.  An id outside [0, num_blocks) reads nothing and writes 0.
// It moves the bytes paged decode attention reads, with no compute, as the
// measured ceiling its rate is compared with.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kCopyThreads) void read_blocks_kernel(ReadBlocksArgs a) {
    __shared__ uint32_t part[kCopyThreads / 64];
    const int64_t b = a.ids[blockIdx.x];
    uint32_t x = 0;
    if (b >= 0 && b < a.num_blocks) {
        const int64_t base = b * a.block_stride + a.layer_off;
        const char *k = a.k + base;
        const char *v = a.v ? a.v + base : nullptr;
        const int n16 = (int)(a.slice_bytes >> 4);
        for (int i0 = threadIdx.x; i0 < n16; i0 += kCopyThreads * kUnroll) {
            u32x4 kk[kUnroll], vv[kUnroll];
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) {
                const int i = i0 + u * kCopyThreads;
                kk[u] = i < n16 ? ld16_stream(k + ((int64_t)i << 4)) : u32x4{0, 0, 0, 0};
                vv[u] = (v && i < n16) ? ld16_stream(v + ((int64_t)i << 4)) : u32x4{0, 0, 0, 0};
            }
#pragma unroll
            for (int u = 0; u < kUnroll; ++u) x ^= kk[u].x ^ kk[u].y ^ kk[u].z ^ kk[u].w ^
                                                     vv[u].x ^ vv[u].y ^ vv[u].z ^ vv[u].w;
        }
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) x ^= (uint32_t)__shfl_xor((int)x, d);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t r = 0;
#pragma unroll
        for (int wv = 0; wv < kCopyThreads / 64; ++wv) r ^= part[wv];
        a.out[blockIdx.x] = r;
    }
}

hipError_t launch_read_blocks(const ReadBlocksArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(read_blocks_kernel, dim3((unsigned)a.n), dim3(kCopyThreads), 0, s, a);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Contract validation (debug): counts offsets outside [0, bs), seq_len
// outside [0, min(capacity, max_seq_len)] with capacity = bt_stride*bs - off
// [P3 sec. 2.2], used table entries outside [0, num_blocks), and slots that
// are neither -1 nor inside the pool [P2 sec. 2.2].
// ---------------------------------------------------------------------------
__global__ void zero_u64_kernel(unsigned long long *p) {
    if (threadIdx.x == 0 && blockIdx.x == 0) *p = 0ull;
}

__global__ __launch_bounds__(256) void validate_kernel(ValidateArgs a) {
    unsigned long long bad = 0;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // per sequence: offset and length against the table's capacity
    for (int64_t s = tid; s < a.num_seqs; s += nthreads) {
        const int64_t off = a.offsets[s];
        const int64_t L = a.seq_lens[s];
        if (off < 0 || off >= a.block_size) ++bad;
        const int64_t cap = (int64_t)a.bt_stride * a.block_size - off;
        if (L < 0 || L > cap || (a.max_seq_len >= 0 && L > a.max_seq_len)) ++bad;
    }
    // per used table entry: (seq, j) with j <= (off + L - 1) / bs
    const int64_t pairs = (int64_t)a.num_seqs * a.bt_stride;
    for (int64_t k = tid; k < pairs; k += nthreads) {
        const int64_t s = k / a.bt_stride;
        const int64_t j = k - s * a.bt_stride;
        const int64_t off = a.offsets[s];
        const int64_t L = a.seq_lens[s];
        if (off >= 0 && off < a.block_size && L > 0 && j <= (off + L - 1) / a.block_size) {
            const int32_t b = a.block_tables[k];
            if (b < 0 || b >= a.num_blocks) ++bad;
        }
    }
    for (int64_t i = tid; i < a.num_tokens; i += nthreads) {
        const int64_t sl = a.slots[i];
        if (sl != -1 && (sl < 0 || sl >= a.total_slots)) ++bad;
    }
    if (bad) atomicAdd(a.count, bad);
}

// Clears n 32-bit words (counters that a kernel expects to start at zero);
// a fill kernel rather than hipMemsetAsync, so a captured graph holds no
// memset node.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t *p, int64_t n) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t launch_zero_words(uint32_t *p, int64_t n, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 1024) blocks = 1024;
    hipLaunchKernelGGL(zero_words_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

hipError_t launch_validate(const ValidateArgs &a, hipStream_t s) {
    hipLaunchKernelGGL(zero_u64_kernel, dim3(1), dim3(64), 0, s, a.count);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int64_t work = (int64_t)a.num_seqs * a.bt_stride;
    if (work < a.num_tokens) work = a.num_tokens;
    if (work < a.num_seqs) work = a.num_seqs;
    int64_t blocks = (work + 255) / 256;
    if (blocks < 1) blocks = 1;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(validate_kernel, dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pkv
