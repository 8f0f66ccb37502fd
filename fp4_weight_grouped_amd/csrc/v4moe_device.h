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

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// fp32 -> OCP E4M3 byte: nearest value, ties to even mantissa, magnitudes at or
// beyond 464 (half an ulp above 448) saturate to +-448, never NaN.  Works on
// the fp32 bit pattern: normal results keep the top 3 mantissa bits with
// round-to-nearest-even on the 20 dropped bits (a carry moves into the
// exponent field); results below 2^-6 are multiples of 2^-9.
__device__ __forceinline__ uint32_t e4m3_rne_sat(float v)
{
    uint32_t u = __float_as_uint(v);
    uint32_t sign = (u >> 24) & 0x80u;
    uint32_t a = u & 0x7FFFFFFFu;
    if (a >= 0x43E80000u)                         // |v| >= 464
        return sign | 0x7Eu;
    if (a < 0x3C800000u) {                        // |v| < 2^-6
        float s = __uint_as_float(a) * 512.0f;    // exact scaling, in [0, 8)
        return sign | (uint32_t)__builtin_rintf(s);
    }
    uint32_t q = ((((a >> 23) - 127u + 7u)) << 3) | ((a >> 20) & 7u);
    uint32_t rem = a & 0xFFFFFu;
    q += (rem > 0x80000u) | ((rem == 0x80000u) & (q & 1u));
    q = q > 0x7Eu ? 0x7Eu : q;
    return sign | q;
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
