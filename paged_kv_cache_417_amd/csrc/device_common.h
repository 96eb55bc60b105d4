// device_common.h — vector types and small device helpers for gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace pa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte global load/store through a vector type (one dwordx4 per lane).
__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }
__device__ __forceinline__ void st16(void *p, u32x4 v) { *reinterpret_cast<u32x4 *>(p) = v; }
// 16-byte load marked nontemporal: the K/V stream of a decode call is read
// once, and the hint keeps it from displacing cache lines that are reused.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// 8-byte global loads (one dwordx2 per lane), plain and nontemporal.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ u32x2 ld8(const void *p) { return *reinterpret_cast<const u32x2 *>(p); }
__device__ __forceinline__ u32x2 ld8_nt(const void *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2 *>(p));
}

// Eight OCP E4M3 codes (bytes of w, lowest first) -> eight bf16 values, in
// order, two codes per v_cvt_scalef32_pk_bf16_fp8 with scale 1.  Exact: an
// E4M3 value has at most four significant bits and lies within bf16's
// range, so no rounding happens anywhere.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 w) {
    u32x4 r;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        r[2 * h] = __builtin_bit_cast(uint32_t,
                                      __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.f, false));
        r[2 * h + 1] = __builtin_bit_cast(
            uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[h], 1.f, true));
    }
    return r;
}

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Wave64 butterfly exchange (ds_bpermute under the hood for cross-row masks).
__device__ __forceinline__ float xor_shuffle(float v, int mask) { return __shfl_xor(v, mask, 64); }

// Max / sum over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48),
// on the VALU.  v_permlane16_swap(a, b) leaves rows (a0, b0, a2, b2) in a and
// (a1, b1, a3, b3) in b; v_permlane32_swap(a, b) leaves (a_lo, b_lo) and
// (a_hi, b_hi).  With a = b = v, combining a and b pairs every lane with its
// partner row; two swaps cover all four rows.  Written as inline assembly on
// two explicit registers: the compiler's builtin for these instructions
// keeps only one of the two results when both operands hold the same value.
// The s_nop pairs give the VALU-write -> permlane-read wait states.
__device__ __forceinline__ void swap16(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(float &a, float &b) {
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float rows4_max(float v) {
    float a = v, b = v;
    swap16(a, b);
    float c = fmaxf(a, b), d = c;
    swap32(c, d);
    return fmaxf(c, d);
}
__device__ __forceinline__ float rows4_sum(float v) {
    float a = v, b = v;
    swap16(a, b);
    float c = a + b, d = c;
    swap32(c, d);
    return c + d;
}

// DPP moves within a 16-lane row.  Controls: quad_perm [1,0,3,2] = 0xB1,
// quad_perm [2,3,0,1] = 0x4E, row_half_mirror = 0x141, row_mirror = 0x140.
template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(
        0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}

// Sum over groups of N adjacent lanes (N in 2, 4, 8, 16); every lane of the
// group ends with the group total.  Pairing: xor 1, xor 2 inside a quad,
// then mirrors, which pair each lane with a lane of the other half.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    static_assert(N == 2 || N == 4 || N == 8 || N == 16, "group size");
    v += dpp<0xB1>(v);
    if constexpr (N >= 4) v += dpp<0x4E>(v);
    if constexpr (N >= 8) v += dpp<0x141>(v);
    if constexpr (N >= 16) v += dpp<0x140>(v);
    return v;
}

constexpr float kNegInf = -__builtin_inff();

// 2^x on the transcendental unit (v_exp_f32), without the library's
// rescaling for subnormal results: those flush to zero.  Softmax weights
// below 2^-126 of the running maximum change nothing.  2^0 = 1 and
// 2^-inf = 0 exactly.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// MFMA k-slot -> head-dim map shared by the A and B operands of a
// v_mfma_f32_16x16x32_bf16 contraction over head dims: k-step ks, lane group
// g (= lane / 16) covers the 8 dims starting at the returned offset, so each
// lane reads 32 contiguous bytes per 64-dim slab.  Any map works as long as
// both operands use the same one.
__device__ __forceinline__ int kslot_dim(int ks, int g) {
    return 64 * (ks >> 1) + 16 * g + 8 * (ks & 1);
}

// Work item of one decode workgroup.  The grid is 1-D over
// kv_head (fastest) x sequence x slot (slowest).  Consecutive workgroups go
// to the eight XCDs in turn, so with the kv head fastest each XCD receives
// the same share of heads of every sequence and slot -- equal work per XCD
// whatever the length mix.  Slots count partitions back from the end of a
// sequence: the last slot holds every sequence's final, usually partial,
// partition, so the shortest work is dispatched last and the kernel drains
// with short waves (decode_partition() turns a slot into a partition).
struct DecodeItem {
    int kvh, seq, slot;
};
__device__ __forceinline__ DecodeItem decode_item(uint32_t i, int num_kv_heads, int num_seqs) {
    const uint32_t rest = i / (uint32_t)num_kv_heads;
    return DecodeItem{(int)(i - rest * (uint32_t)num_kv_heads),
                      (int)(rest % (uint32_t)num_seqs), (int)(rest / (uint32_t)num_seqs)};
}
// Partition of a slot for a sequence with np of at most np_max partitions;
// negative when the sequence has no partition in that slot.
__device__ __forceinline__ int decode_partition(int slot, int np, int np_max) {
    return np - np_max + slot;
}

}  // namespace pa
