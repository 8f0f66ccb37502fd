// v4moe_device.h -- device-side number formats and fragment helpers for gfx950.
//
// Sources (cited by short tag and section):
//   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
//   P4 = "DeepSeek-V4 的暗线之二：训练一台不会失控的万亿参数机器"
// Number formats: OCP MX v1.0 (E2M1, E8M0) and OCP OFP8 (E4M3, "FN" flavour).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace v4moe {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// bf16 bits -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// fp32 pair -> two bf16 (a in the low half), round to nearest even
// (v_cvt_pk_bf16_f32; equal to rounding the fp32 bit pattern for every finite
// input).
__device__ __forceinline__ uint32_t bf16x2(float a, float b)
{
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    const bf2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// fp32 pair -> two OCP E4M3 bytes (a in the low byte): nearest value, ties to
// even, magnitudes beyond 448 saturate to +-448, never NaN.  gfx950's
// v_cvt_pk_fp8_f32 rounds to nearest even but turns overflow into NaN, so the
// inputs are clamped to +-448 first (a value that rounds to 448 stays 448).
__device__ __forceinline__ uint32_t e4m3x2(float a, float b)
{
    a = __builtin_amdgcn_fmed3f(a, -448.0f, 448.0f);
    b = __builtin_amdgcn_fmed3f(b, -448.0f, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}

// Four fp32 values -> four OCP E2M1 codes, a in bits 0-3 ... d in bits 12-15:
// nearest value, ties to the even code, magnitudes from 6 up saturate to 6, the
// sign kept (a negative value that rounds to zero gives code 8).  gfx950's
// v_cvt_scalef32_pk_fp4_f32 with scale 1.0 does exactly this for every
// non-NaN fp32 input.
__device__ __forceinline__ uint32_t e2m1x4(float a, float b, float c, float d)
{
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, a, b, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, c, d, 1.0f, 1);
    return r & 0xFFFFu;
}

// SiLU(g) * u with the hardware exp2 and reciprocal (about 2 ulp; the result
// is requantised to E4M3 right after).
__device__ __forceinline__ float silu_mul(float g, float u)
{
    const float e = __builtin_amdgcn_exp2f(-g * 1.44269504088896341f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// 16x16 output tile over one 128-wide K chunk on gfx950's block-scaled
// matrix cores (v_mfma_scale_f32_16x16x128_f8f6f4): A = E4M3 activations with
// scale 1 (E8M0 127), B = E2M1 weight codes, each lane's 32 codes scaled by
// 2^(sb_byte - 127), sb_byte = byte SEL of sb.  The hardware multiplies the
// exact values e4m3(a) * e2m1(w) * 2^b; inside the window b in [-8, 6] every
// e2m1(w) * 2^b is itself an E4M3 value (P1 §4: the FP4 -> FP8 conversion is
// lossless), so the products are those of an FP8 x FP8 GEMM over the
// dequantised weights, without materialising the E4M3 bytes.
// Lane layouts (g = l/16):
//   A: lane l holds row l%16; dwords 0-3 = K 16g..16g+15, dwords 4-7 = K
//      64+16g..64+16g+15 of the chunk, one byte per element in K order;
//   B: lane l holds column l%16 and K 32g..32g+31: element k in byte k/2, the
//      low nibble for even k (four dwords);
//   C: lane l holds rows 4g+i, i = 0..3, of column l%16.
template <int SEL>
__device__ __forceinline__ v4f mfma_e4m3_e2m1(v8i a, uint4 b, int sb)
{
    const v8i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, bv, z, 0, 4, 0, 127, SEL, sb);
}
// The same instruction with the operands swapped: A = E2M1 weight codes (lane l:
// weight row l%16, K 32(l/16)..+31, its E8M0 byte SEL of sw as scale), B = E4M3
// activations (lane l: token l%16, the split K layout of A above).  Result:
// lane l holds weight rows 4(l/16)+i, i = 0..3, for token l%16.
template <int SEL>
__device__ __forceinline__ v4f mfma_e2m1_e4m3(uint4 w, int sw, v8i x)
{
    const v8i wv = {(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, x, z, 4, 0, SEL, sw, 0, 127);
}
__device__ __forceinline__ v4f mfma_e2m1_e4m3_sel(int sel, uint4 w, int sw, v8i x)
{
    switch (sel & 3) {   // sel is a constant after unrolling: one instruction remains
    case 0: return mfma_e2m1_e4m3<0>(w, sw, x);
    case 1: return mfma_e2m1_e4m3<1>(w, sw, x);
    case 2: return mfma_e2m1_e4m3<2>(w, sw, x);
    default: return mfma_e2m1_e4m3<3>(w, sw, x);
    }
}

__device__ __forceinline__ v4f mfma_e4m3_e2m1_sel(int sel, v8i a, uint4 b, int sb)
{
    switch (sel & 3) {   // sel is a constant after unrolling: one instruction remains
    case 0: return mfma_e4m3_e2m1<0>(a, b, sb);
    case 1: return mfma_e4m3_e2m1<1>(a, b, sb);
    case 2: return mfma_e4m3_e2m1<2>(a, b, sb);
    default: return mfma_e4m3_e2m1<3>(a, b, sb);
    }
}

// splitmix64 output function (Steele, Lea & Flood, OOPSLA 2014).
__device__ __forceinline__ uint64_t splitmix64(uint64_t v)
{
    uint64_t z = v + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

}  // namespace v4moe
