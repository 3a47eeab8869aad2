// Device helpers for the gfx950 (CDNA4) paged-attention kernels.
//
// Wave64 conventions used by every kernel in this library.  A lane l is
// split into r = l & 15 (row / column index of a 16x16 MFMA tile) and
// c = l >> 4 (one of four lane groups).  For the 16x16xK MFMAs used here:
//   A operand  lane (r, c) supplies row r, k-slots of group c
//   B operand  lane (r, c) supplies column r, k-slots of group c
//   D result   lane (r, c) holds D[4c + e][r], e = 0..3
// Which k each (group, element) slot stands for is the same for A and B, so a
// kernel may map contraction indices to slots in any order as long as both
// operands agree; the kernels use that freedom to keep every lane's global
// loads 16 bytes wide and contiguous.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Online softmax keeps a column's running max until a block raises it by
// more than this many log2 units; weights then stay below 2^8, far inside
// fp32 and bf16 range, and the normalisation uses the same weights, so the
// result is unchanged up to rounding.  A larger jump rescales, which leaves
// the new maximum's weight exactly exp2(0) = 1.
constexpr float kRescaleLog2 = 8.0f;

enum KvKind { KV_F32 = 0, KV_BF16 = 1, KV_FP8 = 2 };

template <class To, class From>
__device__ __forceinline__ To bitcast(const From& x) {
    static_assert(sizeof(To) == sizeof(From), "bitcast size");
    return __builtin_bit_cast(To, x);
}

// ---------------------------------------------------------------------------
// cross-lane reductions over the four lane groups (lanes r, r+16, r+32, r+48)
// using the gfx950 row-swap permutes (plain VALU ops, no LDS traffic).
// ---------------------------------------------------------------------------
__device__ __forceinline__ float group_max4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float group_sum4(float x) {
    auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// 4x4 transpose of 32-bit words over the four lane groups: on entry group c
// holds x[0..3]; on exit slot j of group c holds what was x[c] of group j.
// permlane32_swap exchanges the upper lane half of its first operand with the
// lower half of its second, permlane16_swap the odd 16-lane rows of the first
// with the even rows of the second: the first pass moves the off-diagonal
// 2x2 word blocks between the halves, the second transposes each 2x2 block.
__device__ __forceinline__ void group_transpose4(unsigned x[4]) {
#pragma unroll
    for (int jl = 0; jl < 2; ++jl) {
        const auto p = __builtin_amdgcn_permlane32_swap(x[jl], x[2 + jl], false, false);
        x[jl] = p[0];
        x[2 + jl] = p[1];
    }
#pragma unroll
    for (int jh = 0; jh < 2; ++jh) {
        const auto p = __builtin_amdgcn_permlane16_swap(x[2 * jh], x[2 * jh + 1], false, false);
        x[2 * jh] = p[0];
        x[2 * jh + 1] = p[1];
    }
}

// Maximum over the 16 lanes of one row (same c), by xor shuffles.
__device__ __forceinline__ float row_max16(float x) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
    return x;
}


// hardware exp2 / log2 (v_exp_f32, v_log_f32)
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// ---------------------------------------------------------------------------
// conversions
// ---------------------------------------------------------------------------
// two fp32 -> packed bf16 (round to nearest even, hardware convert)
__device__ __forceinline__ unsigned pack_bf16x2(float lo, float hi) {
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return bitcast<unsigned>(v);
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(unsigned w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }

// four OCP e4m3fn codes (one dword) -> four bf16 (exact; 1.0 scale)
__device__ __forceinline__ u32x2 fp8x4_to_bf16x4(unsigned w) {
    bf16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    bf16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true);
    u32x2 r;
    r.x = bitcast<unsigned>(lo);
    r.y = bitcast<unsigned>(hi);
    return r;
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------
// D(16x16) += A(16x32) B(32x16), bf16 inputs, fp32 accumulate
__device__ __forceinline__ f32x4 mfma_16x16x32_bf16(u32x4 a, u32x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(bitcast<bf16x8>(a), bitcast<bf16x8>(b), acc,
                                                   0, 0, 0);
}

// D(16x16) += A(16x16) B(16x16), bf16 inputs, fp32 accumulate
__device__ __forceinline__ f32x4 mfma_16x16x16_bf16(u32x2 a, u32x2 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bitcast<i16x4>(a), bitcast<i16x4>(b), acc,
                                                     0, 0, 0);
}

// D(16x16) += A(16x4) B(4x16), fp32
__device__ __forceinline__ f32x4 mfma_16x16x4_f32(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }


// 16-byte / 8-byte global loads (plain vector loads)
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x2 ld8(const void* p) { return *reinterpret_cast<const u32x2*>(p); }

// loads of KV data, which every kernel reads exactly once: non-temporal, so
// the stream of K/V tiles does not evict what is reused (tables, q, partials)
#ifndef PA_KV_NONTEMPORAL
#define PA_KV_NONTEMPORAL 1
#endif
__device__ __forceinline__ u32x4 ldkv16(const void* p) {
#if PA_KV_NONTEMPORAL
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#else
    return ld16(p);
#endif
}
__device__ __forceinline__ u32x2 ldkv8(const void* p) {
#if PA_KV_NONTEMPORAL
    return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
#else
    return ld8(p);
#endif
}

}  // namespace pa
