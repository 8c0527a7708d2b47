// Matrix-core helpers shared by the grouped-query decode and the prefill kernels: 16-bit operand
// types, the MFMA shapes used (16x16x32 for the logits, 16x16x16 for the weighted sum), packing of
// fp32 weights into 16-bit operand pairs, and the lane-group reductions of the output layout
// (lane l = 16 g + n holds rows 4g .. 4g+3 of column n).
#pragma once

#include "attention.h"

namespace pkv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <class E>
struct Mfma;

template <>
struct Mfma<F16> {
    static __device__ inline f32x4 mma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                      0, 0, 0);
    }
    static __device__ inline f32x4 mma16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0,
                                                     0, 0);
    }
    static __device__ inline unsigned short bits(float x) {
        const _Float16 h = static_cast<_Float16>(x);  // round to nearest even
        return __builtin_bit_cast(unsigned short, h);
    }
    static __device__ inline float value(unsigned short b) {
        return static_cast<float>(__builtin_bit_cast(_Float16, b));
    }
    // the fp32 values of the low and high halves of a packed word
    static __device__ inline float lo(unsigned w) { return value(static_cast<unsigned short>(w & 0xffffu)); }
    static __device__ inline float hi(unsigned w) { return value(static_cast<unsigned short>(w >> 16)); }
    static __device__ inline unsigned pack2(float lo, float hi) {
        const f16x2 v = {static_cast<_Float16>(lo), static_cast<_Float16>(hi)};  // round to nearest even
        return __builtin_bit_cast(unsigned, v);
    }
    // acc + the two packed values (exact products by one, fp32 accumulation)
    static __device__ inline float sum2(unsigned packed, float acc) {
        const f16x2 ones = {static_cast<_Float16>(1.f), static_cast<_Float16>(1.f)};
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
    }
};

template <>
struct Mfma<BF16> {
    static __device__ inline f32x4 mma(const u32x4 &a, const u32x4 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                       c, 0, 0, 0);
    }
    static __device__ inline f32x4 mma16(const u32x2 &a, const u32x2 &b, const f32x4 &c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                         0, 0, 0);
    }
    static __device__ inline unsigned short bits(float x) {
        const __bf16 h = static_cast<__bf16>(x);  // round to nearest even
        return __builtin_bit_cast(unsigned short, h);
    }
    static __device__ inline float value(unsigned short b) { return __uint_as_float(static_cast<unsigned>(b) << 16); }
    // the fp32 values of the low and high halves of a packed word: each half moved to (or left
    // at) the top of a word, one instruction
    static __device__ inline float lo(unsigned w) {
        // bytes 1, 0 of w over two zero bytes (a byte permute: a shift of a packed conversion's
        // result is otherwise rebuilt from a second conversion)
        return __uint_as_float(__builtin_amdgcn_perm(0u, w, 0x01000c0cu));
    }
    static __device__ inline float hi(unsigned w) { return __uint_as_float(w & 0xffff0000u); }
    static __device__ inline unsigned pack2(float lo, float hi) {
        const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};  // round to nearest even
        return __builtin_bit_cast(unsigned, v);
    }
    static __device__ inline float sum2(unsigned packed, float acc) {
        const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
    }
};

// Max over lanes l, l^16, l^32, l^48 (the four lane groups), in every lane: permlane swaps,
// no LDS round trip.
__device__ inline float max_over_lane_groups(float x) {
    const unsigned u = __float_as_uint(x);
    const auto a = __builtin_amdgcn_permlane32_swap(u, u, false, false);  // lanes l and l^32
    const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const unsigned v = __float_as_uint(y);
    const auto b = __builtin_amdgcn_permlane16_swap(v, v, false, false);  // lanes l and l^16
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ inline unsigned word(const u32x4 &r, int w) {
    return w == 0 ? r.x : (w == 1 ? r.y : (w == 2 ? r.z : r.w));
}

// Transposed LDS read (ds_read_b64_tr_b16): every lane addresses 8 bytes (four 16-bit values);
// within each group of 16 lanes, lane r receives as its element j the element r % 4 of the four
// that lane 4j + r / 4 of the group addressed. With lane (n, g) of a group addressing row
// r0 + 4g + n / 4, columns c0 + 4 (n % 4) .. + 3 of a row-major 16-bit tile, lane (n, g) receives
// column c0 + n of rows r0 + 4g .. r0 + 4g + 3: a column of the tile, as an MFMA operand wants it.
__device__ inline u32x2 lds_read_tr16(const void *p) {
    const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)p);
    return __builtin_bit_cast(u32x2, v);
}

// s_waitcnt lgkmcnt(0) alone (vmcnt and expcnt at their maxima): before a barrier that orders LDS
// work only, so global loads stay in flight and global stores need not complete.
constexpr int kWaitLgkm0 = 0xC07F;

// Table entries as scalar loads: the constant address space (the tables are not written while
// a kernel runs) with a uniform index gives s_load, whose completion counter is not the one the
// K/V loads use, so looking an entry up never waits for K/V data.
typedef const __attribute__((address_space(4))) int32_t TableEntry;

}  // namespace pkv
