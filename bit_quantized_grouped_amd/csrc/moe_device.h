// Device-side building blocks for gfx950 (CDNA4): vector types, bf16
// packing, the 4-bit dequantization of one code word, MFMA and wave helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moeq4 {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    bf16x2_t r;
    r[0] = (__bf16)lo;
    r[1] = (__bf16)hi;
    return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}

// A 4-bit code q held alone in a byte reads, as an fp8 e4m3 value, q times a
// fixed power of two (the subnormal step equals the first binade's step, so
// the 16 codes are evenly spaced).  fp8_unit() returns that power of two as
// converted by the hardware; dequantization multiplies by scale / unit,
// which is exact, so fma(q * unit, scale / unit, bias) = fma(q, scale, bias).
__device__ __forceinline__ float fp8_unit() {
    f32x2_t one = __builtin_amdgcn_cvt_pk_f32_fp8(1, false);
    return one[0];
}

// Dequantize one code word (8 consecutive weights along K, lowest k in the
// low nibble) to 8 bf16 in K order: w_i = bf16_rne(fp32(q_i * s + b)).
// s_scaled = s / fp8_unit().
__device__ __forceinline__ bf16x8_t dequant_word(uint32_t w, float s_scaled, float b) {
    const uint32_t lo = w & 0x0F0F0F0Fu;         // codes 0, 2, 4, 6 in bytes 0..3
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;  // codes 1, 3, 5, 7
    const f32x2_t q02 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, false);
    const f32x2_t q46 = __builtin_amdgcn_cvt_pk_f32_fp8((int)lo, true);
    const f32x2_t q13 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, false);
    const f32x2_t q57 = __builtin_amdgcn_cvt_pk_f32_fp8((int)hi, true);
    u32x4_t r;
    r[0] = pack_bf16x2(__builtin_fmaf(q02[0], s_scaled, b), __builtin_fmaf(q13[0], s_scaled, b));
    r[1] = pack_bf16x2(__builtin_fmaf(q02[1], s_scaled, b), __builtin_fmaf(q13[1], s_scaled, b));
    r[2] = pack_bf16x2(__builtin_fmaf(q46[0], s_scaled, b), __builtin_fmaf(q57[0], s_scaled, b));
    r[3] = pack_bf16x2(__builtin_fmaf(q46[1], s_scaled, b), __builtin_fmaf(q57[1], s_scaled, b));
    return __builtin_bit_cast(bf16x8_t, r);
}

// Offset, in words, of code word c (weights 8c .. 8c+7) of row n of one
// expert's [N, K] code matrix.  Layout 0 is row-major; layout 1 stores, per
// tile of 64 rows and per 64 K, the tile's rows together (16-row groups of
// 16 rows x 8 words), so a tile's K-chunk is one contiguous block.  Four
// consecutive words c .. c+3 with c % 4 == 0 are contiguous in both.
__device__ __forceinline__ uint32_t code_word(int layout, uint32_t n, uint32_t c, uint32_t K) {
    if (layout == 0) return n * (K / 8) + c;
    return ((n / 64) * (K / 64) + c / 8) * 512 + ((n % 64) / 16) * 128 + (n % 16) * 8 + c % 8;
}

// D = A(16x32) * B(32x16) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%16][8*(l/16) .. +8] and B[8*(l/16) .. +8][l%16];
// it holds D[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4_t mfma_16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// D = A(32x16) * B(16x32) + C, bf16 inputs, fp32 accumulate.
// Lane l supplies A[l%32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l%32]; it
// holds D[8*(i/4) + 4*(l/32) + i%4][l%32], i = 0..15.  Only the pairing of A
// and B elements along K matters: a caller may assign each lane's 8 K
// positions freely as long as its A and B elements follow the same order.
__device__ __forceinline__ f32x16_t mfma_32x32x16(bf16x8_t a, bf16x8_t b, f32x16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// z * sigmoid(z) with the hardware exp2 and reciprocal (about 1 ulp each).
__device__ __forceinline__ float silu_f32(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * z));
}

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int mask) {
    return __shfl_xor(v, mask, WAVE);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moeq4
