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
//   A work item is (sequence, kv head, split): split j covers logical tokens
//   [j*S, (j+1)*S).  One wavefront (64 lanes) owns one work item and all G
//   query heads of its kv head, so each K/V row is read from HBM once and
//   used G times.  A workgroup holds up to 4 wavefronts = 4 kv heads of the
//   same (sequence, split): they share the block-table entries, which are
//   staged in LDS once per workgroup, and read neighbouring 256-byte head
//   segments of the same token rows.
//
// Lane layout ("row layout")
//   A kv-head row of one token is D*E bytes = LPR lanes x 16 bytes.  Lane
//   (r, c) = (lane / LPR, lane % LPR) loads piece c of the row of token
//   chunk_base + i*RPI + r for pass i (RPI = 64/LPR rows per wavefront
//   instruction), so every load instruction covers RPI whole rows.
//   QK:  partial dot over the lane's VEC elements (v_dot2_f32_bf16 for
//        bf16), then an all-reduce over the LPR lanes of the row with DPP
//        (quad_perm, row_half_mirror, row_mirror): every lane of the row
//        ends with the same fp32 score.
//   softmax: scores are kept in the exp2 domain (scale*log2 e folded in);
//        per 16-token chunk the wavefront takes one max per query head
//        (shared by all lanes), so m is wave-uniform; l and the P.V
//        accumulators are per-lane partials over the lane's own rows and are
//        summed across row groups once at the end.
//   PV:  acc[g][e] += p * V[row][c*VEC + e] in fp32.
//   Masked tokens (past seq_len, or an invalid table entry) get score -inf
//   and are never loaded, so poisoned (NaN) pool slots cannot leak in.
//
// Split-K: with more than one split per sequence, each work item writes its
// unnormalised (m, l, acc) to the workspace and a second kernel merges the
// splits of each (sequence, query head) in split order:
//   M = max_j m_j,  L = sum_j l_j 2^(m_j - M),  O = sum_j acc_j 2^(m_j - M) / L.
// With one split the first kernel normalises and writes the output itself.
#include "pkv_internal.h"

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

template <int DT>
struct Elem;
template <>
struct Elem<0> {  // PKV_F32
    static constexpr int kBytes = 4;
};
template <>
struct Elem<1> {  // PKV_BF16
    static constexpr int kBytes = 2;
};

__device__ __forceinline__ u32x4 ld16(const char *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even float -> bf16 bits (quiet NaN kept NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// A 32-bit word as a pair of bf16.  The word is passed by value on
// purpose: applying __builtin_bit_cast directly to an ext_vector element
// (q.y, q.z, ...) makes this compiler read element .x every time.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Dot product of one 16-byte piece of q with one 16-byte piece of K.
template <int DT>
__device__ __forceinline__ float dot16(u32x4 q, u32x4 k);

template <>
__device__ __forceinline__ float dot16<1>(u32x4 q, u32x4 k) {
    float s = 0.0f;
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.x), as_bf16x2(k.x), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.y), as_bf16x2(k.y), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.z), as_bf16x2(k.z), s, false);
    s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(q.w), as_bf16x2(k.w), s, false);
    return s;
}

template <>
__device__ __forceinline__ float dot16<0>(u32x4 q, u32x4 k) {
    float s = __uint_as_float(q.x) * __uint_as_float(k.x);
    s = fmaf(__uint_as_float(q.y), __uint_as_float(k.y), s);
    s = fmaf(__uint_as_float(q.z), __uint_as_float(k.z), s);
    s = fmaf(__uint_as_float(q.w), __uint_as_float(k.w), s);
    return s;
}

// The VEC fp32 values of one 16-byte piece.
template <int DT>
__device__ __forceinline__ void unpack16(u32x4 x, float *f);

template <>
__device__ __forceinline__ void unpack16<1>(u32x4 x, float *f) {
    f[0] = bf16_lo(x.x); f[1] = bf16_hi(x.x);
    f[2] = bf16_lo(x.y); f[3] = bf16_hi(x.y);
    f[4] = bf16_lo(x.z); f[5] = bf16_hi(x.z);
    f[6] = bf16_lo(x.w); f[7] = bf16_hi(x.w);
}

template <>
__device__ __forceinline__ void unpack16<0>(u32x4 x, float *f) {
    f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
    f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
}

// Store VEC fp32 values as one 16-byte piece of the output dtype.
template <int DT>
__device__ __forceinline__ void store16(char *p, const float *f);

template <>
__device__ __forceinline__ void store16<1>(char *p, const float *f) {
    u32x4 x;
    x.x = f32_to_bf16_bits(f[0]) | (f32_to_bf16_bits(f[1]) << 16);
    x.y = f32_to_bf16_bits(f[2]) | (f32_to_bf16_bits(f[3]) << 16);
    x.z = f32_to_bf16_bits(f[4]) | (f32_to_bf16_bits(f[5]) << 16);
    x.w = f32_to_bf16_bits(f[6]) | (f32_to_bf16_bits(f[7]) << 16);
    *reinterpret_cast<u32x4 *>(p) = x;
}

template <>
__device__ __forceinline__ void store16<0>(char *p, const float *f) {
    u32x4 x;
    x.x = __float_as_uint(f[0]); x.y = __float_as_uint(f[1]);
    x.z = __float_as_uint(f[2]); x.w = __float_as_uint(f[3]);
    *reinterpret_cast<u32x4 *>(p) = x;
}

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over the W consecutive lanes of a row group (W a power of two <= 64);
// every lane of the group gets the same bits (each step adds two equal
// partial sums in both orders, and fp addition commutes).
template <int W>
__device__ __forceinline__ float row_allsum(float v) {
    if constexpr (W >= 2) v += dpp<0xB1>(v);   // quad_perm [1,0,3,2]
    if constexpr (W >= 4) v += dpp<0x4E>(v);   // quad_perm [2,3,0,1]
    if constexpr (W >= 8) v += dpp<0x141>(v);  // row_half_mirror
    if constexpr (W >= 16) v += dpp<0x140>(v); // row_mirror
    if constexpr (W >= 32) v += __shfl_xor(v, 16);
    if constexpr (W >= 64) v += __shfl_xor(v, 32);
    return v;
}

// Reduce across the row groups of a wavefront (lanes equal mod W).
template <int W>
__device__ __forceinline__ float cross_rows_max(float v) {
#pragma unroll
    for (int m = W; m < 64; m <<= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}
template <int W>
__device__ __forceinline__ float cross_rows_sum(float v) {
#pragma unroll
    for (int m = W; m < 64; m <<= 1) v += __shfl_xor(v, m);
    return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

template <int DT, int D, int G>
__global__ __launch_bounds__(256) void decode_kernel(DecodeArgs a) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int VEC = 16 / E;               // elements per 16-byte piece
    constexpr int LPR = D / VEC;              // lanes per kv-head row
    constexpr int RPI = 64 / LPR;             // rows per wavefront pass
    constexpr int NP = kChunkTokens / RPI;    // passes per chunk
    static_assert(LPR >= 4 && LPR <= 64 && RPI <= kChunkTokens, "head_dim out of range");
    constexpr float kNegInf = -__builtin_huge_valf();

    __shared__ int32_t bt_s[kBtLds];

    // Workgroups are dealt round-robin to the 8 XCDs; renumber them so that
    // consecutive logical items (same head group and split, consecutive
    // sequences: a shared prefix is read by neighbours) share an XCD's L2.
    const int nwg = gridDim.x;
    const int bid = blockIdx.x;
    const int xcd = bid & 7;
    const int per = nwg >> 3, rem = nwg & 7;
    const int lid = xcd * per + min(xcd, rem) + (bid >> 3);
    const int seq = lid % a.num_seqs;
    const int rest = lid / a.num_seqs;
    const int split = rest % a.max_splits;
    const int hg = rest / a.max_splits;

    const int L = a.seq_lens[seq];
    const int t0 = split * a.split_tokens;
    const bool direct = a.max_splits == 1;
    if (!direct && t0 >= L) return;  // this split is empty (uniform per workgroup)
    const int t1 = min(L, t0 + a.split_tokens);
    const int64_t off = a.offsets[seq];
    const int lbs = a.pool.lbs;
    const int64_t bsm = (1ll << lbs) - 1;
    const int64_t jb0 = (off + t0) >> lbs;
    const int nbt = t1 > t0 ? (int)(((off + t1 - 1) >> lbs) - jb0 + 1) : 0;
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

    const int w = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int h = hg * a.heads_per_wg + w;
    if (h >= a.num_kv_heads) return;
    const int r = lane / LPR;
    const int c = lane % LPR;
    const int hq0 = h * G;

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

    for (int tc = t0; tc < t1; tc += kChunkTokens) {
        u32x4 kx[NP], vx[NP];
        bool ok[NP];
#pragma unroll
        for (int i = 0; i < NP; ++i) {
            const int t = tc + i * RPI + r;
            ok[i] = false;
            kx[i] = u32x4{0, 0, 0, 0};
            vx[i] = u32x4{0, 0, 0, 0};
            if (t < t1) {
                const int64_t p = off + t;
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
    if (r != 0) return;

    if (direct) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float o[VEC];
#pragma unroll
            for (int e = 0; e < VEC; ++e) o[e] = l[g] > 0.0f ? acc[g][e] / l[g] : 0.0f;
            store16<DT>(a.out + (((int64_t)seq * a.num_q_heads + hq0 + g) * D + c * VEC) * E, o);
        }
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t item = ((int64_t)seq * a.max_splits + split) * a.num_q_heads + hq0 + g;
            float *wa = a.ws_acc + item * D + c * VEC;
#pragma unroll
            for (int e = 0; e < VEC; e += 4)
                *reinterpret_cast<float4 *>(wa + e) =
                    make_float4(acc[g][e], acc[g][e + 1], acc[g][e + 2], acc[g][e + 3]);
            if (c == 0) *reinterpret_cast<float2 *>(a.ws_ml + item * 2) = make_float2(m[g], l[g]);
        }
    }
}

// Second pass: merge the splits of one (sequence, query head).
template <int DT, int D>
__global__ __launch_bounds__(64) void reduce_kernel(DecodeArgs a) {
    constexpr int E = Elem<DT>::kBytes;
    constexpr int DPT = D / 64;  // elements per lane
    constexpr float kNegInf = -__builtin_huge_valf();
    const int seq = blockIdx.x / a.num_q_heads;
    const int hq = blockIdx.x - seq * a.num_q_heads;
    const int64_t L = a.seq_lens[seq];
    int64_t ns = L > 0 ? (L + a.split_tokens - 1) / a.split_tokens : 0;
    if (ns > a.max_splits) ns = a.max_splits;
    const int64_t item0 = (int64_t)seq * a.max_splits * a.num_q_heads + hq;
    const int64_t step = a.num_q_heads;

    float M = kNegInf;
    for (int64_t j = 0; j < ns; ++j) M = fmaxf(M, a.ws_ml[(item0 + j * step) * 2]);
    float den = 0.0f;
    float o[DPT];
#pragma unroll
    for (int k = 0; k < DPT; ++k) o[k] = 0.0f;
    for (int64_t j = 0; j < ns; ++j) {
        const int64_t item = item0 + j * step;
        const float mj = a.ws_ml[item * 2];
        const float lj = a.ws_ml[item * 2 + 1];
        const float wj = mj == kNegInf ? 0.0f : fast_exp2(mj - M);
        den = fmaf(lj, wj, den);
        const float *src = a.ws_acc + item * D + threadIdx.x * DPT;
#pragma unroll
        for (int k = 0; k < DPT; ++k) o[k] = fmaf(src[k], wj, o[k]);
    }
    char *dst = a.out + (((int64_t)seq * a.num_q_heads + hq) * D + threadIdx.x * DPT) * E;
#pragma unroll
    for (int k = 0; k < DPT; ++k) {
        const float v = den > 0.0f ? o[k] / den : 0.0f;
        if constexpr (DT == 1) {
            reinterpret_cast<uint16_t *>(dst)[k] = (uint16_t)f32_to_bf16_bits(v);
        } else {
            reinterpret_cast<float *>(dst)[k] = v;
        }
    }
}

template <int DT, int D, int G>
static hipError_t run_decode(const DecodeArgs &a, hipStream_t s) {
    const int64_t nwg = (int64_t)a.head_groups * a.max_splits * a.num_seqs;
    hipLaunchKernelGGL((decode_kernel<DT, D, G>), dim3((unsigned)nwg), dim3(64 * a.heads_per_wg),
                       0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || a.max_splits == 1) return e;
    hipLaunchKernelGGL((reduce_kernel<DT, D>), dim3((unsigned)((int64_t)a.num_seqs * a.num_q_heads)),
                       dim3(64), 0, s, a);
    return hipGetLastError();
}

typedef hipError_t (*DecodeFn)(const DecodeArgs &, hipStream_t);

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

}  // namespace pkv
