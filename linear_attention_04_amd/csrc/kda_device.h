// kda_device.h -- device helpers shared by the gfx950 KDA kernels.
//
// Lane layouts used throughout (one 64-lane wave, lane l, c = l & 15, grp = l >> 4):
//  * accumulator ("D") layout of a 16x16 MFMA tile: lane l holds rows 4*grp + i
//    (i = 0..3) of column c;
//  * A operand of v_mfma_f32_16x16x16_bf16: lane l holds row c, reduction indices
//    4*grp + i; B operand: column c, reduction indices 4*grp + i. A D-layout tile
//    converted to bf16 is therefore directly a B operand;
//  * A / B operands of v_mfma_f32_16x16x32_bf16: row (A) or column (B) c, eight
//    reduction indices per lane. Which eight the hardware pairs is irrelevant as
//    long as A and B use the same (lane group, element) -> index assignment, which
//    the kernels guarantee by building both operands from the same channel set.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// The key (channel) order the kernels share. In the row layout (lane = token c), element
// e of lane group grp holds channel chan_of(e, grp): eight consecutive channels per
// 16-byte load of a bf16 row. Row r of 16 x 16 accumulator tile m of a 128-key state
// slice holds key key_of(m, r). The two agree, key_of(m, 4 grp + i) = chan_of(4 m + i,
// grp), so a state tile in the accumulator layout, rounded to bf16, pairs key by key
// with row-layout operands in a 16x16x32 product (elements 8s .. 8s + 7 = tiles 2s, 2s + 1).
__host__ __device__ constexpr int chan_of(int e, int grp) { return 32 * (e >> 3) + 8 * grp + (e & 7); }
__host__ __device__ constexpr int key_of(int m, int r) {
    return 32 * (m >> 1) + 8 * (r >> 2) + 4 * (m & 1) + (r & 3);
}

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_16x16x16(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 as_s16x4(bf16x4 x) { return __builtin_bit_cast(s16x4, x); }

// Round-to-nearest-even fp32 -> bf16 (hardware conversion on gfx950).
__device__ __forceinline__ __bf16 to_bf16(float x) { return static_cast<__bf16>(x); }
__device__ __forceinline__ float from_bf16(__bf16 x) { return static_cast<float>(x); }

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
    bf16x4 r;
    r[0] = to_bf16(x[0]); r[1] = to_bf16(x[1]); r[2] = to_bf16(x[2]); r[3] = to_bf16(x[3]);
    return r;
}

// Two fp32 values rounded to a packed bf16 pair (one v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned int pack_bf16x2(float a, float b) {
    bf16x2 p;
    p[0] = to_bf16(a);
    p[1] = to_bf16(b);
    return __builtin_bit_cast(unsigned int, p);
}

// (a, b) = hi + lo with hi = bf16(a, b), lo = bf16((a, b) - hi): ~16 significant
// bits in two packed bf16 pairs, three VALU operations per value.
__device__ __forceinline__ void split_pair(float a, float b, unsigned int &hi, unsigned int &lo) {
    unsigned int h = pack_bf16x2(a, b);
    asm volatile("" : "+v"(h));  // reuse the packed word for both halves (no second conversion)
    hi = h;
    lo = pack_bf16x2(a - __uint_as_float(h << 16), b - __uint_as_float(h & 0xffff0000u));
}

// x = hi + lo for four values.
__device__ __forceinline__ void split_bf16x4(f32x4 x, bf16x4 &hi, bf16x4 &lo) {
    uint2 h, l;
    split_pair(x[0], x[1], h.x, l.x);
    split_pair(x[2], x[3], h.y, l.y);
    hi = __builtin_bit_cast(bf16x4, h);
    lo = __builtin_bit_cast(bf16x4, l);
}

// DPP: value of lane (l - N) within the same 16-lane row, or 0 where that lane is
// outside the row.
template <int N>
__device__ __forceinline__ float row_shr(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x110 + N, 0xf, 0xf, false));
}

// DPP: value of lane N of this lane's 16-lane row. Every source lane exists, so
// bound_ctrl (zero for a missing source) changes nothing here; it lets the compiler
// fold the move into the instruction that uses it.
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x150 + N, 0xf, 0xf, true));
}

// DPP: value of lane (l + N) within the same 16-lane row, or 0 where that lane is
// outside the row.
template <int N>
__device__ __forceinline__ float row_shl(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x100 + N, 0xf, 0xf, false));
}

// Inclusive suffix sum over the 16 lanes of each row (lane c gets x_c + ... + x_15).
__device__ __forceinline__ float row_suffix_sum(float x) {
    x += row_shl<1>(x);
    x += row_shl<2>(x);
    x += row_shl<4>(x);
    x += row_shl<8>(x);
    return x;
}

// Inclusive prefix sum over the 16 lanes of each row (lane c gets x_0 + ... + x_c).
__device__ __forceinline__ float row_inclusive_sum(float x) {
    x += row_shr<1>(x);
    x += row_shr<2>(x);
    x += row_shr<4>(x);
    x += row_shr<8>(x);
    return x;
}

// Map a linear workgroup id so that the workgroups of one unit of data share an XCD:
// the dispatcher deals workgroups to the device's `xccs` XCDs round robin
// (id % xccs), so the `per_unit` workgroups that share one unit (e.g. the value
// tiles of one head) are placed at ids unit_slot + xccs * k and all run behind one
// L2. The grid holds a multiple of xccs units.
__device__ __forceinline__ void xcd_unit_split(int id, int per_unit, int xccs, int &unit, int &member) {
    const int xcd = id % xccs;
    const int rest = id / xccs;
    member = rest % per_unit;
    unit = (rest / per_unit) * xccs + xcd;
}

}  // namespace kda
