// attn_common.h -- device helpers shared by the attention kernels
// (kernels_decode.hip, kernels_prefill.hip): vector types, bf16 <-> fp32
// conversions, 16-byte dot products, cross-lane reductions, the direct
// global -> LDS copy, and the tile geometry of the bf16 matrix-core path.
// Everything here is inline or a template.
#pragma once

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

// Two floats as a bf16 pair (lo in bits 0..15), rounded to nearest even by
// the gfx950 packed conversion (v_cvt_pk_bf16_f32; NaN stays NaN).
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
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

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Two finite floats as a bf16 pair, round to nearest even (one
// v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

constexpr float kNegInf = -__builtin_huge_valf();

#ifndef PKV_DECODE_RING
#define PKV_DECODE_RING 3
#endif
// Pipeline depth of the bf16 decode kernel (chunks in flight + the one
// being computed).
constexpr int kDecodeRing = PKV_DECODE_RING;

// Copy 16 bytes per lane from global memory straight into LDS: lane i's
// bytes land at lds_wave_base + 16*i (global_load_lds_dwordx4).  The LDS
// address must be the same in every lane.
__device__ __forceinline__ void lds_copy16(const char *src, char *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(const_cast<char *>(src),
                                     (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0, 0);
}

// Nontemporal reads (global_load ... nt) of pool bytes that one call reads
// once.  Measured on MI355X (same process, decode_mfma / decode_q8 kernels,
// microseconds without -> with the hint):
//   bf16 V, global -> LDS (lds_copy16_nt): decode batch 42.5 -> 40.5,
//     prefix sharing 96.6 -> 95.0, long context 192.2 -> 168.9;
//   bf16 K, global -> registers: prefix sharing 96.6 -> 110.9 (the prefix
//     that 64 sequences share is re-fetched), long context 192.2 -> 174.7;
//     so bf16 K loads stay ordinary;
//   int8 codes and scales (ld16_nt): decode batch 30.8 -> 29.4, long
//     context 112.1 -> 102.8, prefix sharing level (66.8 / 67.4).
// A plain 1 GiB read in 64 KiB pieces per workgroup moves 5.85 TB/s with
// ordinary loads and 6.65 TB/s with the hint.
__device__ __forceinline__ u32x4 ld16_nt(const char *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// lds_copy16 with the nontemporal hint.
__device__ __forceinline__ void lds_copy16_nt(const char *src, char *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(const_cast<char *>(src),
                                     (__attribute__((address_space(3))) void *)lds_wave_base, 16, 0,
                                     2 /* nt */);
}

// LDS reads issued from inline asm, complete (lgkmcnt(0)) when the block
// ends.  Why: the compiler cannot tell which LDS bytes a global -> LDS copy
// writes, and before an LDS read it cannot separate from the copies in
// flight it waits for all of them (vmcnt(0)), prefetches issued for later
// stages included, which puts a whole memory latency into every stage.
// Kernels using these order each read after the copies it depends on
// themselves (an s_waitcnt on their own copies, then a barrier).
__device__ __forceinline__ uint32_t lds_addr(const char *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char *)p;
}

// 16-byte reads (ds_read_b128) at p + S * k, k = 0 .. 7.
template <int S>
__device__ __forceinline__ void lds_read16_x8(const char *p, u32x4 (&r)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:%9\n\t"
        "ds_read_b128 %2, %8 offset:%10\n\t"
        "ds_read_b128 %3, %8 offset:%11\n\t"
        "ds_read_b128 %4, %8 offset:%12\n\t"
        "ds_read_b128 %5, %8 offset:%13\n\t"
        "ds_read_b128 %6, %8 offset:%14\n\t"
        "ds_read_b128 %7, %8 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lds_addr(p)), "i"(S), "i"(2 * S), "i"(3 * S), "i"(4 * S), "i"(5 * S), "i"(6 * S), "i"(7 * S)
        : "memory");
}

// 16-byte reads (ds_read_b128) at p + S * k, k = 0 .. 3.
template <int S>
__device__ __forceinline__ void lds_read16_x4(const char *p, u32x4 (&r)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %4 offset:%5\n\t"
        "ds_read_b128 %2, %4 offset:%6\n\t"
        "ds_read_b128 %3, %4 offset:%7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3])
        : "v"(lds_addr(p)), "i"(S), "i"(2 * S), "i"(3 * S)
        : "memory");
}

// Transposed reads (ds_read_b64_tr_b16: the B-operand layout of a 16x16x32
// MFMA from 4 rows of 8 bytes) at p + S * k and p + T + S * k, k = 0 .. 3,
// into r[k] and r[4 + k].
template <int S, int T>
__device__ __forceinline__ void lds_read_tr16_x8(const char *p, uint64_t (&r)[8]) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %8 offset:%9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:%10\n\t"
        "ds_read_b64_tr_b16 %3, %8 offset:%11\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:%12\n\t"
        "ds_read_b64_tr_b16 %5, %8 offset:%13\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:%14\n\t"
        "ds_read_b64_tr_b16 %7, %8 offset:%15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]), "=&v"(r[7])
        : "v"(lds_addr(p)), "i"(S), "i"(2 * S), "i"(3 * S), "i"(T), "i"(T + S), "i"(T + 2 * S), "i"(T + 3 * S)
        : "memory");
}

// Keep the compiler from moving LDS accesses across this point; the LDS
// unit itself serves one wavefront's requests in order.
__device__ __forceinline__ void wave_lds_order() {
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
}

// max(v of lane l, v of lane l ^ 16) and the same for l ^ 32, with the
// gfx950 row swaps (v_permlane16_swap / v_permlane32_swap: VALU operations,
// no LDS permute in the dependency chain).  With both operands v, the
// 16-swap leaves lane l holding its own value in one result and that of
// lane l ^ 16 in the other; likewise for 32.
__device__ __forceinline__ float max_xor16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v of lane l plus v of lane l ^ 16 (then ^ 32), with the row swaps; both
// lanes of a pair get the same bits.
__device__ __forceinline__ float sum_xor16(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float v) {
    const unsigned u = __float_as_uint(v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Max and sum over all 64 lanes, the result in every lane: DPP within rows
// of 16 lanes, then the row swaps across rows -- all VALU, no LDS permute
// round trip in the chain.  Every lane gets the same bits (each step
// combines two equal partial results in both orders).
__device__ __forceinline__ float wave_max(float x) {
    x = fmaxf(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
    x = fmaxf(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
    x = fmaxf(x, dpp<0x141>(x));  // row_half_mirror
    x = fmaxf(x, dpp<0x140>(x));  // row_mirror
    return max_xor32(max_xor16(x));
}

__device__ __forceinline__ float wave_sum(float x) {
    x = row_allsum<16>(x);
    const unsigned u = __float_as_uint(x);
    const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    x = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
    const unsigned v = __float_as_uint(x);
    const auto r32 = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}

__device__ __forceinline__ float lane_value(float x, int lane) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

template <int D>
struct MfmaShape {
    static constexpr int E = 2;
    static constexpr int ROWB = D * E;           // bytes of one kv-head row
    static constexpr int PPR = ROWB / 16;        // 16-byte pieces per row
    static constexpr int RPI = 64 / PPR;         // rows per tile-load instruction
    static constexpr int NP = 16 / RPI;          // tile-load instructions per chunk
    static constexpr int KS = D / 32;            // QK^T steps (k = 32)
    static constexpr int NV = D / 16;            // P.V column slabs (n = 16)
    static constexpr int VSLAB = 1024 + 32;      // one tile-load instruction + padding
    static constexpr int VTILE = NP * VSLAB;     // V tile of one ring slot
    static constexpr int KROW = ROWB + 16;       // padded K-tile row
    static constexpr int KTILE = 16 * KROW;
    static constexpr int NSLOT = kDecodeRing;    // pipeline stages (chunks in flight + 1)
    static constexpr int LOADS = KS + NP;        // vector-memory ops per chunk (K in operand layout, V rows)
    static_assert(D % 32 == 0 && PPR >= 4 && PPR <= 16 && RPI * ROWB == 1024, "shape");
};

}  // namespace pkv
