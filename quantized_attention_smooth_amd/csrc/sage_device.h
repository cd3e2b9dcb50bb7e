// sage_device.h -- device-side definitions shared by the gfx950 kernels of
// the quantized attention forward (quantize passes and the attention kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <hip/hip_bf16.h>
#include <stdint.h>

#include "sage_kernels.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

// MFMA accumulator bias: the int32 QK^T accumulators start at the bit pattern
// of fp32 1/(2 pi), 0x3E22F983, whose mantissa field is M = 0x22F983.  For
// -M <= S < 2^23 - M the accumulated integer stays in the binade [1/8, 1/4),
// so read as an fp32 it is exactly (K + S) * 2^-26 with K = 2^23 + M =
// 10680707: no int -> float conversion is needed, and the row factor carries
// the 2^26 (kAccScale).  |S| <= 128 * 127 * 127 = 2064512 < M for
// head_dim <= 128.  gfx950 encodes 1/(2 pi) as an inline constant, so the
// first MFMA of a score chain takes the bias without a register.
constexpr int kAccBiasBits = 0x3E22F983;
constexpr float kAccBias = 0x1.45F306p-3f;              // the same bits as an fp32 (K * 2^-26)
constexpr float kAccScale = 0x1p26f;
constexpr int kNegInfBits = (int)0xFF800000u;   // -inf; smallest signed int32 of any score

__device__ __forceinline__ float bits_f(int x) { return __int_as_float(x); }

// fp16/bf16 element helpers -------------------------------------------------
// (conversions from fp32 round to nearest even)
template <bool BF16> struct Half;
template <> struct Half<false> {
    __device__ static float to_f(uint16_t b) { return (float)__builtin_bit_cast(_Float16, b); }
    __device__ static uint16_t from_f(float x) { return __builtin_bit_cast(uint16_t, (_Float16)x); }
};
template <> struct Half<true> {
    __device__ static float to_f(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }
    __device__ static uint16_t from_f(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
};

// The 8 fp16 or bf16 values packed in 16 bytes, as fp32 (exact).
template <bool BF16>
__device__ __forceinline__ void unpack8(const uint4& raw, float v[8]) {
    const uint16_t* e = reinterpret_cast<const uint16_t*>(&raw);
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = Half<BF16>::to_f(e[j]);
}

// Order of keys inside an aligned block of 64 in the transposed V operand:
// position 32*h + 16*b + 4*r + e holds key 32*b + 8*r + 4*h + e.  This is the
// order in which a lane of the S^T = K Q^T accumulator holds its keys (lane
// half h, accumulator block b, register i = 4*r + e), so that the softmax
// output feeds the P.V MFMA as its B operand without any data movement.
__device__ __forceinline__ int v_perm_pos(int key64) {
    int b = key64 >> 5, r = (key64 >> 3) & 3, h = (key64 >> 2) & 1, e = key64 & 3;
    return (h << 5) | (b << 4) | (r << 2) | e;
}

// LDS 16-byte-chunk swizzles for ds_read_b128 of 32 consecutive rows at one
// logical chunk: rows that fall into the same 256-byte bank window must hit
// different chunks.  K tile rows hold Dp bytes; V^T tile rows hold 64 keys
// (64 B for FP8, 128 B for fp16/bf16).
template <int ROW_BYTES>
__device__ __forceinline__ int swz(int row, int chunk) {
    if constexpr (ROW_BYTES >= 128) return chunk ^ ((row >> 1) & 7);
    else return chunk ^ ((row >> 2) & 3);
}

__device__ __forceinline__ int xcd_remap(int bid, int nwg) {
    // Workgroups are dispatched round-robin over the 8 XCDs.  Renumber them so
    // that consecutive logical ids (query tiles of the same head) run on the
    // same XCD and share its L2 for the K/V stream.
    const int per = nwg / 8, rem = nwg % 8;
    const int xcd = bid % 8, idx = bid / 8;
    return (xcd < rem) ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

__device__ __forceinline__ float swap_half_max(float x) {
    // max over lanes l and l ^ 32; x is never NaN here, so the plain
    // instruction serves (fmaxf would first quiet both operands)
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__int_as_float(r[0])), "v"(__int_as_float(r[1])));
    return m;
}
__device__ __forceinline__ float swap_half_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_int(x), __float_as_int(x), false, false);
    return __int_as_float(r[0]) + __int_as_float(r[1]);
}

// INT8 quantization of Q and K (the quantize pass and the attention kernel's
// own quantization of Q share these, so that both give the same bits).
// A group with absolute maximum amax has scale amax / 127 and multiplier
// fl(127 / amax), each one correctly rounded division (both 0 for an
// all-zero group).
__device__ __forceinline__ void int8_group_scale(float amax, float& scale, float& inv) {
    scale = amax > 0.f ? amax / 127.0f : 0.f;
    inv = amax > 0.f ? 127.0f / amax : 0.f;
}
// The codes rint(fl(x * inv)) of 8 values as 8 bytes, first value in the low
// byte.  Adding 1.5 * 2^23 rounds fl(x * inv) to an integer (ties to even)
// held in the low bits of the sum, whose low byte is the code in two's
// complement; with |x| <= amax, |fl(x * inv)| < 127.5, so no clamp is needed.
// Product and sum are rounded separately (never one fused operation).
__device__ __forceinline__ uint2 int8_codes8(const float (&x)[8], float inv) {
#pragma clang fp contract(off)
    constexpr float kRound = 12582912.0f;
    uint32_t c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __float_as_uint(x[j] * inv + kRound);
    const uint32_t w0 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c[3], c[2], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c[1], c[0], 0x0c0c0400u), 0x05040100u);
    const uint32_t w1 = __builtin_amdgcn_perm(__builtin_amdgcn_perm(c[7], c[6], 0x0c0c0400u),
                                              __builtin_amdgcn_perm(c[5], c[4], 0x0c0c0400u), 0x05040100u);
    return make_uint2(w0, w1);
}

}  // namespace sage
