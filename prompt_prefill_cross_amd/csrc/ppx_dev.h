// Device-side helpers shared by the engine's kernels (gfx950, wave64).
#pragma once

#include "ppx_internal.h"

namespace ppx {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef float f4 __attribute__((ext_vector_type(4)));

// Fragment-tiled fp16 activation layout, the A operand of every row-batched
// GEMM.  A[M][K] is cut into 16-row x 32-column tiles of 1 KB, stored
// tile-row-major; inside a tile, lane l = r % 16 + 16 * ((k % 32) / 8) holds
// the eight consecutive k of its row (the v_mfma_f32_16x16x32_f16 A-operand
// order), so one 16-byte load per lane fetches a whole fragment from 1 KB of
// contiguous memory.  Rows are padded to a multiple of 16 in the allocation.
__device__ __forceinline__ size_t tiled_index(int r, int k, int K) {
    return (((size_t)(r >> 4) * (unsigned)(K >> 5) + (unsigned)(k >> 5)) * 64 + (r & 15) + 16 * ((k >> 3) & 3)) * 8 +
           (k & 7);
}

__device__ __forceinline__ f4 mfma16(const h8 &a, const h8 &b, const f4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// (x & 0x000F000F) | 0x64006400 in one v_and_or_b32.  Both constants live in
// VGPRs: gfx950's VOP3 encoding reads at most one scalar or literal operand,
// so with two literals the compiler falls back to a separate AND and OR.
__device__ __forceinline__ uint32_t q4_pair_bits(uint32_t x) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "v"(0x000F000Fu), "v"(0x64006400u));
    return r;
}

// Eight codes of one repacked word -> fp16 d*(code-8), rounded to nearest even.
// (w >> 4i) & 0x000F000F | 0x6400_6400 is the fp16 pair (1024+q_{2i}, 1024+q_{2i+1});
// subtracting 1032 is exact, the product with d rounds once.
__device__ __forceinline__ h8 q4_word_to_h8(uint32_t w, _Float16 d) {
    h8 r;
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
    const h2 dd = {d, d};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h2 v = __builtin_bit_cast(h2, q4_pair_bits(w >> (4 * i)));
        v = (v - bias) * dd;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

// (code - 8) exactly, as fp16, for the eight codes of a repacked word.
__device__ __forceinline__ h8 q4_word_codes(uint32_t w) {
    h8 r;
    const h2 bias = {(_Float16)1032.0f, (_Float16)1032.0f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        h2 v = __builtin_bit_cast(h2, q4_pair_bits(w >> (4 * i))) - bias;
        r[2 * i] = v[0];
        r[2 * i + 1] = v[1];
    }
    return r;
}

// Code of element e (0..7) in a repacked word.
__device__ __forceinline__ int q4_word_code(uint32_t w, int e) {
    int sh = (e & 1) ? (16 + 4 * (e >> 1)) : (4 * (e >> 1));
    return (int)((w >> sh) & 15u);
}

// Exact fp32 weight W[n][k] of a repacked matrix.
__device__ __forceinline__ float q4r_weight(const Q4R &w, int n, int k) {
    const int kc = k >> 6, s = (k >> 5) & 1, g = (k >> 3) & 3, e = k & 7;
    const int grp = n >> 4, col = n & 15;
    const size_t base = (size_t)grp * (w.K >> 6) + kc;
    const uint32_t word = w.nib[(base * 64 + g * 16 + col) * 2 + s];
    const float d = __half2float(w.scl[(base * 16 + col) * 2 + s]);
    return d * (float)(q4_word_code(word, e) - 8);
}

// Exact fp32 value of column c of a raw Q4_0 row (18-byte blocks).
__device__ __forceinline__ float q4_raw_weight(const uint8_t *row, int c) {
    const uint8_t *b = row + (size_t)(c >> 5) * 18;
    const int j = c & 31;
    const uint16_t dbits = (uint16_t)b[0] | ((uint16_t)b[1] << 8);
    const float d = __half2float(__ushort_as_half(dbits));
    const uint8_t byte = b[2 + (j & 15)];
    const int q = (j < 16) ? (byte & 15) : (byte >> 4);
    return d * (float)(q - 8);
}

// z * sigmoid(t) with the hardware base-2 exponential and reciprocal (about
// 1 ulp each): e^-t = 2^(-t log2 e).  For t -> -inf the exponential overflows
// to +inf and the product goes to -0, the limit.
__device__ __forceinline__ float mul_sigmoid(float z, float t) {
    const float e = __builtin_amdgcn_exp2f(-1.4426950408889634f * t);
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// GELU, tanh form: 0.5 z (1 + tanh(u)) = z * sigmoid(2u), u = sqrt(2/pi) (z + 0.044715 z^3).
__device__ __forceinline__ float gelu_tanh_f(float z) {
    const float k0 = 0.7978845608028654f;  // sqrt(2/pi)
    return mul_sigmoid(z, 2.0f * k0 * (z + 0.044715f * z * z * z));
}

__device__ __forceinline__ float silu_f(float z) { return mul_sigmoid(z, z); }

__device__ __forceinline__ float act_f(int act, float g) {
    return act == ACT_GEGLU ? gelu_tanh_f(g) : silu_f(g);
}

// Cross-lane exchanges on VALU, without a trip through the LDS queue.
// swap32 / swap16 (gfx950 v_permlane32_swap / v_permlane16_swap, both
// operands the same register) give each lane its own value and that of lane
// l ^ 32 / l ^ 16, in some order; row_ror<k> gives the value of lane
// (i + k) mod 16 within each row of 16 lanes (DPP), which for k = 8 is lane i ^ 8.
struct LanePair {
    float a, b;
};
__device__ __forceinline__ LanePair swap32(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ LanePair swap16(float v) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return {__uint_as_float(r[0]), __uint_as_float(r[1])};
}
template <int K>
__device__ __forceinline__ float row_ror(float v) {
    static_assert(K >= 1 && K <= 15, "row rotation");
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x120 + K, 0xf, 0xf, false));
}

// Reduction over the wave in the order of the xor butterfly (distance 32,
// 16, 8, 4, 2, 1): after the folds at distances above 2^k every lane holds
// the same value as the lanes that differ from it in the higher bits of its
// row, so the rotation partner (i + 2^k) mod 16 holds what lane i ^ 2^k
// holds, and each lane ends with the butterfly's result, bit for bit.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op) {
    LanePair p = swap32(v);
    v = op(p.a, p.b);
    p = swap16(v);
    v = op(p.a, p.b);
    v = op(v, row_ror<8>(v));
    v = op(v, row_ror<4>(v));
    v = op(v, row_ror<2>(v));
    return op(v, row_ror<1>(v));
}

__device__ __forceinline__ float wave_sum(float v) {
    return wave_reduce(v, [](float x, float y) { return x + y; });
}

__device__ __forceinline__ float wave_max(float v) {
    return wave_reduce(v, [](float x, float y) { return fmaxf(x, y); });
}

}  // namespace ppx
