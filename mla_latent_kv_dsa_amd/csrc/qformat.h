// qformat.h -- decoding of the quantized kv_b formats on the vector ALU.
// aiknowledge.cn Ch.7 sec. 03, sec. 3 and 5: int8 / FP8 / MXFP4 weight formats, each a bounded-loss
// form of the same weights; colibri-analysis 06 "MLA attention and KV cache", sec. 2.3: the absorbed
// path reads kv_b only in its two per-head products, over such rows.
//
// A quantized kv_b is [rows][L] (rows = heads x (qk_nope + v_head), L = kv_lora):
//   MLA_Q_FP8_E4M3  one byte per weight, OCP E4M3 (no infinities), one fp32 scale per row
//   MLA_Q_INT8      one signed byte per weight, one fp32 scale per row
//   MLA_Q_MXFP4     OCP MX: FP4 E2M1, two per byte (even column in the low nibble), an E8M0
//                   scale byte per 32 columns
// Format 0 below stands for the plain bf16 kv_b.  A byte code without its row scale, and an MXFP4
// weight with its block scale, is exact in bf16: at most eight significant bits, and for block
// scales 2^-127 .. 2^125 an exponent inside bf16's range (subnormal at the low end).
#pragma once
#include "common.h"

namespace mla {

// The codes are decoded by gfx950's scaled conversions (v_cvt_scalef32_pk_*): two E4M3 codes of a
// 16-bit half, or the two E2M1 codes of a byte (the even column in the low nibble), to two fp32 or
// two bf16 values, multiplied by a power of two given as the exponent field of an fp32 operand (an
// E8M0 scale byte x is the fp32 bit pattern x << 23; x = 0 stands for 2^-127).  The E4M3 NaN codes
// (S.1111.111) give NaN.  Byte codes and MXFP4 weights are exact in either type.
typedef __bf16 q_bf16x2_t __attribute__((ext_vector_type(2)));
typedef float q_f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float q_scale_e8m0(uint32_t x) { return __uint_as_float(x << 23); }

template <bool HI> __device__ __forceinline__ uint32_t q_e4m3x2_bf16(uint32_t w)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
template <int BYTE> __device__ __forceinline__ uint32_t q_e2m1x2_bf16(uint32_t w, float scale)
{
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, scale, BYTE));
}
template <bool HI> __device__ __forceinline__ q_f32x2_t q_e4m3x2_f32(uint32_t w)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(w, 1.0f, HI);
}
template <int BYTE> __device__ __forceinline__ q_f32x2_t q_e2m1x2_f32(uint32_t w, float scale)
{
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, scale, BYTE);
}

// An int8 code pair (bytes 0 and 1 of w) as two bf16 (exact: at most 8 significant bits)
__device__ __forceinline__ uint32_t q_i8x2_bf16(uint32_t w)
{
    const float lo = (float)(int8_t)(w & 255u), hi = (float)(int8_t)((w >> 8) & 255u);
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xffff0000u);
}

// Weights row, columns c .. c + 3 (c a multiple of 4) of a quantized [rows][L] matrix, scaled.
template <int FMT>
__device__ __forceinline__ void q_load4(const uint8_t *__restrict__ codes, const void *__restrict__ scales, int64_t row,
                                        int L, int c, float (&w)[4])
{
    if constexpr (FMT == MLA_Q_MXFP4) {
        const uint32_t v = *reinterpret_cast<const uint16_t *>(codes + row * (L / 2) + c / 2);
        const float sc = q_scale_e8m0(reinterpret_cast<const uint8_t *>(scales)[row * (L / 32) + c / 32]);
        const q_f32x2_t a = q_e2m1x2_f32<0>(v, sc), b = q_e2m1x2_f32<1>(v, sc);
        w[0] = a[0]; w[1] = a[1]; w[2] = b[0]; w[3] = b[1];
    } else {
        const uint32_t v = *reinterpret_cast<const uint32_t *>(codes + row * L + c);
        const float sc = reinterpret_cast<const float *>(scales)[row];
        if constexpr (FMT == MLA_Q_FP8_E4M3) {
            const q_f32x2_t a = q_e4m3x2_f32<false>(v), b = q_e4m3x2_f32<true>(v);
            w[0] = sc * a[0]; w[1] = sc * a[1]; w[2] = sc * b[0]; w[3] = sc * b[1];
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = sc * (float)(int8_t)((v >> (8 * k)) & 255u);
        }
    }
}

// Raw weights of 8 consecutive columns c .. c + 7 (c a multiple of 8) of one row, loaded first and
// decoded later (so the loads of many rows can be in flight together).
template <int FMT> struct QRaw8;
template <> struct QRaw8<0> { uint4 v; };                                   // 8 bf16
template <> struct QRaw8<MLA_Q_FP8_E4M3> { uint2 v; float s; };             // 8 codes + row scale
template <> struct QRaw8<MLA_Q_INT8> { uint2 v; float s; };
template <> struct QRaw8<MLA_Q_MXFP4> { uint32_t v; uint32_t s; };          // 8 nibbles + block scale

// w: the bf16 kv_b (FMT 0) or the codes; scales unused for FMT 0
template <int FMT>
__device__ __forceinline__ QRaw8<FMT> q_raw8(const void *__restrict__ w, const void *__restrict__ scales, int64_t row,
                                             int L, int c)
{
    QRaw8<FMT> r;
    if constexpr (FMT == 0) {
        // read once per call: nontemporal (decode step 42.2 -> 42.0 us, three alternating pairs)
        typedef unsigned int u4v __attribute__((ext_vector_type(4)));
        const u4v x = __builtin_nontemporal_load(reinterpret_cast<const u4v *>(reinterpret_cast<const bf16_t *>(w) + row * L + c));
        r.v = make_uint4(x.x, x.y, x.z, x.w);
    } else if constexpr (FMT == MLA_Q_MXFP4) {
        r.v = *reinterpret_cast<const uint32_t *>(reinterpret_cast<const uint8_t *>(w) + row * (L / 2) + c / 2);
        r.s = reinterpret_cast<const uint8_t *>(scales)[row * (L / 32) + c / 32];
    } else {
        r.v = *reinterpret_cast<const uint2 *>(reinterpret_cast<const uint8_t *>(w) + row * L + c);
        r.s = reinterpret_cast<const float *>(scales)[row];
    }
    return r;
}

// The 8 raw weights as 8 exact bf16 values w and a factor s with weight = s * w: the byte codes
// and their row scale, the MXFP4 weights with their block scale applied (s = 1), bf16 as it is.
template <int FMT> __device__ __forceinline__ void q_bf16x8(const QRaw8<FMT> &r, uint4 &w, float &s)
{
    if constexpr (FMT == 0) {
        w = r.v;
        s = 1.f;
    } else if constexpr (FMT == MLA_Q_MXFP4) {
        const float sc = q_scale_e8m0(r.s);
        w = make_uint4(q_e2m1x2_bf16<0>(r.v, sc), q_e2m1x2_bf16<1>(r.v, sc), q_e2m1x2_bf16<2>(r.v, sc),
                       q_e2m1x2_bf16<3>(r.v, sc));
        s = 1.f;
    } else if constexpr (FMT == MLA_Q_FP8_E4M3) {
        w = make_uint4(q_e4m3x2_bf16<false>(r.v.x), q_e4m3x2_bf16<true>(r.v.x), q_e4m3x2_bf16<false>(r.v.y),
                       q_e4m3x2_bf16<true>(r.v.y));
        s = r.s;
    } else {
        w = make_uint4(q_i8x2_bf16(r.v.x), q_i8x2_bf16(r.v.x >> 16), q_i8x2_bf16(r.v.y), q_i8x2_bf16(r.v.y >> 16));
        s = r.s;
    }
}

// 16 codes of one row (16 bytes, or 8 bytes of MXFP4 with the block scale sc) as 16 bf16 values
template <int FMT> __device__ __forceinline__ void q_bf16x16(const uint4 &c, float sc, uint4 &lo, uint4 &hi)
{
    if constexpr (FMT == MLA_Q_MXFP4) {
        lo = make_uint4(q_e2m1x2_bf16<0>(c.x, sc), q_e2m1x2_bf16<1>(c.x, sc), q_e2m1x2_bf16<2>(c.x, sc),
                        q_e2m1x2_bf16<3>(c.x, sc));
        hi = make_uint4(q_e2m1x2_bf16<0>(c.y, sc), q_e2m1x2_bf16<1>(c.y, sc), q_e2m1x2_bf16<2>(c.y, sc),
                        q_e2m1x2_bf16<3>(c.y, sc));
    } else if constexpr (FMT == MLA_Q_FP8_E4M3) {
        lo = make_uint4(q_e4m3x2_bf16<false>(c.x), q_e4m3x2_bf16<true>(c.x), q_e4m3x2_bf16<false>(c.y),
                        q_e4m3x2_bf16<true>(c.y));
        hi = make_uint4(q_e4m3x2_bf16<false>(c.z), q_e4m3x2_bf16<true>(c.z), q_e4m3x2_bf16<false>(c.w),
                        q_e4m3x2_bf16<true>(c.w));
    } else {
        lo = make_uint4(q_i8x2_bf16(c.x), q_i8x2_bf16(c.x >> 16), q_i8x2_bf16(c.y), q_i8x2_bf16(c.y >> 16));
        hi = make_uint4(q_i8x2_bf16(c.z), q_i8x2_bf16(c.z >> 16), q_i8x2_bf16(c.w), q_i8x2_bf16(c.w >> 16));
    }
}

}  // namespace mla
