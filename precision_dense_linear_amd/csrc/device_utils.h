// Device-side building blocks shared by the FP8 kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// Buffer resource over [base, base + bytes).  Raw (stride 0) buffer loads whose
// offset is at or beyond `bytes` return zero and touch no memory; the kernels
// use this to zero-fill ragged tiles without any out-of-bounds access.
// dword3 0x00020000 is the gfx9 raw 32-bit data format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Offset that is out of range for every resource built with at most 2^31 bytes.
constexpr uint32_t OOB = 0x80000000u;

__device__ __forceinline__ uint32_t clamp_records(int64_t bytes) {
    return bytes <= 0 ? 0u : (bytes >= (int64_t)OOB ? OOB : (uint32_t)bytes);
}

// D = A(32x64) * B(64x32) + C with OCP FP8 operands, FP32 accumulate
// (v_mfma_f32_32x32x64_f8f6f4; zero scale operands select the unscaled
// form).  The operand formats are given per operand: 0 = E4M3, 1 = E5M2 (the
// cbsz / blgp fields select the format of the first / second source).
// Lane l (h = l/32) holds A row l%32 / B column l%32: bytes 0-15 are K
// positions 16h .. 16h+15 of the instruction, bytes 16-31 K positions
// 32+16h .. 32+16h+15 (checked through the scaled form below, whose
// 32-deep K blocks are K 0-31 and 32-63);
// accumulator element r of lane l is row 8*(r/4) + 4*(l/32) + r%4, column l%32.
template <int FMT_SRC0, int FMT_SRC1>
__device__ __forceinline__ v16f mfma_32x32x64_f8(v8i a, v8i b, v16f c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, FMT_SRC0, FMT_SRC1, 0, 0, 0, 0);
}

// The scaled form with E4M3 operands: the products of 32-deep K block b
// (instruction K 0-31 or 32-63) of row / column i are multiplied by
// 2^(e - 127), e the byte BYTE0 (BYTE1) of the scale operand of lane
// 32b + i for the first (second) source (OCP E8M0; the op_sel field picks
// the byte).
template <int BYTE0, int BYTE1>
__device__ __forceinline__ v16f mfma_32x32x64_e4m3_scaled(v8i a, v8i b, v16f c, int e8_src0, int e8_src1) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, BYTE0, e8_src0, BYTE1, e8_src1);
}

// D = A(32x64, 2:4 sparse along K) * B(64x32) + C, E4M3 operands, FP32
// accumulate (v_smfmac_f32_32x32x64_fp8_fp8).  A is given compressed: lane
// l (h = l/32) holds for row l%32 the 16 kept values of instruction K
// 32h .. 32h+31 in K order (two per group of 4), and idx bits 2e .. 2e+1
// give the position (0..3) of kept value e within its group.  B as for the
// dense instruction (bytes 0-15: K 16h..16h+15, 16-31: K 32+16h..), the
// accumulator layout too.  (Both layouts were checked on the GPU against
// the exact product of small-integer operands.)
__device__ __forceinline__ v16f smfmac_32x32x64_e4m3(v4i a_sparse, v8i b, v16f c, int idx) {
    return __builtin_amdgcn_smfmac_f32_32x32x64_fp8_fp8(a_sparse, b, c, idx, 0, 0);
}

// D = A(32x16) * B(16x32) + C in BF16 with FP32 accumulate
// (v_mfma_f32_32x32x16_bf16).  Lane l holds A row l%32 / B column l%32, K
// elements 8*(l/32) .. +7; accumulator layout as for the 32x32x64 form.
// Unlike the FP8 forms (which align each group of 8 products to a 13-bit
// window below the group's largest product and truncate the rest), every
// product of two E4M3 values reaches the FP32 accumulator exactly here.
__device__ __forceinline__ v16f mfma_32x32x16_bf16(v8bf a, v8bf b, v16f c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Eight E4M3 codes (two dwords, code 0 in the low byte) -> eight BF16 values.
// Every E4M3 value is a BF16 value, and the scale is 1, so this is exact
// (v_cvt_scalef32_pk_bf16_fp8, two codes per instruction).
__device__ __forceinline__ v8bf e4m3x8_to_bf16(int lo, int hi) {
    const v2bf r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, false);
    const v2bf r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)lo, 1.0f, true);
    const v2bf r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, false);
    const v2bf r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((unsigned)hi, 1.0f, true);
    return (v8bf){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Eight E5M2 codes -> eight BF16 values, exact as well: every E5M2 value
// (|v| <= 57344, subnormals down to 2^-16) is a BF16 value
// (v_cvt_scalef32_pk_bf16_bf8).
__device__ __forceinline__ v8bf e5m2x8_to_bf16(int lo, int hi) {
    const v2bf r0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((unsigned)lo, 1.0f, false);
    const v2bf r1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((unsigned)lo, 1.0f, true);
    const v2bf r2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((unsigned)hi, 1.0f, false);
    const v2bf r3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_bf8((unsigned)hi, 1.0f, true);
    return (v8bf){r0[0], r0[1], r1[0], r1[1], r2[0], r2[1], r3[0], r3[1]};
}

// Eight codes of format F (0 = E4M3, 1 = E5M2) -> eight BF16 values.
template <int F>
__device__ __forceinline__ v8bf fp8x8_to_bf16(int lo, int hi) {
    if constexpr (F == 0) return e4m3x8_to_bf16(lo, hi);
    else return e5m2x8_to_bf16(lo, hi);
}

// 8-byte LDS transpose read (ds_read_b64_tr_b8).  Within each 16-lane group,
// output lane 8h + c receives byte c of the 8-byte rows addressed by lanes
// 2j + h, j = 0..7 (row j in byte j of the result).
__device__ __forceinline__ v2i lds_read_tr8(const lds_u8* p) {
    return __builtin_amdgcn_ds_read_tr8_b64_v2i32((__attribute__((address_space(3))) v2i*)p);
}

__device__ __forceinline__ v4i lds_read16(const lds_u8* p) {
    return *(const __attribute__((address_space(3))) v4i*)p;
}

// binary32 -> bfloat16, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

// Four binary32 values -> four E4M3 codes (RNE), saturating at +-448: the
// clamp comes first because the converter alone maps |v| > 464 to NaN.
__device__ __forceinline__ uint32_t e4m3x4_sat(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    c = __builtin_amdgcn_fmed3f(c, -448.0f, 448.0f);
    d = __builtin_amdgcn_fmed3f(d, -448.0f, 448.0f);
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint8_t e4m3_sat(float a) {
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_fp8_f32(a, 0.0f, 0, false) & 0xFF);
}

// scale = amax / 448 (IEEE binary32 division); 1 for an all-zero group.
__device__ __forceinline__ float scale_from_amax(float amax) {
    return amax == 0.0f ? 1.0f : __fdiv_rn(amax, 448.0f);
}

// E5M2 counterparts: largest finite value 57344; the clamp keeps values the
// converter would take past the largest finite value (to Inf) at +-57344.
__device__ __forceinline__ uint32_t e5m2x4_sat(float a, float b, float c, float d) {
    a = __builtin_amdgcn_fmed3f(a, -57344.0f, 57344.0f);
    b = __builtin_amdgcn_fmed3f(b, -57344.0f, 57344.0f);
    c = __builtin_amdgcn_fmed3f(c, -57344.0f, 57344.0f);
    d = __builtin_amdgcn_fmed3f(d, -57344.0f, 57344.0f);
    int w = __builtin_amdgcn_cvt_pk_bf8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_bf8_f32(c, d, w, true);
    return (uint32_t)w;
}

__device__ __forceinline__ uint8_t e5m2_sat(float a) {
    a = __builtin_amdgcn_fmed3f(a, -57344.0f, 57344.0f);
    return (uint8_t)(__builtin_amdgcn_cvt_pk_bf8_f32(a, 0.0f, 0, false) & 0xFF);
}

// Format-generic forms (F: 0 = E4M3, 1 = E5M2).
template <int F>
__device__ __forceinline__ uint32_t fp8x4_sat(float a, float b, float c, float d) {
    if constexpr (F == 0) return e4m3x4_sat(a, b, c, d);
    else return e5m2x4_sat(a, b, c, d);
}

template <int F>
__device__ __forceinline__ uint8_t fp8_sat(float a) {
    if constexpr (F == 0) return e4m3_sat(a);
    else return e5m2_sat(a);
}

template <int F>
__device__ __forceinline__ float scale_from_amax_fmt(float amax) {
    return amax == 0.0f ? 1.0f : __fdiv_rn(amax, F == 0 ? 448.0f : 57344.0f);
}

}  // namespace fp8k
