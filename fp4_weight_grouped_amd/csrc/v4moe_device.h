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

// Magnitude of the FP4 E2M1 code m (0..7): 0, 0.5, 1, 1.5, 2, 3, 4, 6.
__device__ __forceinline__ float e2m1_mag(int m)
{
    int e = m >> 1;
    float frac = (m & 1) ? 1.5f : 1.0f;
    return e == 0 ? 0.5f * (float)(m & 1) : ldexpf(frac, e - 1);
}

// Dequantisation table, one entry per E8M0 byte s (sub-block exponent
// b = s - 127): the E4M3 bytes of e2m1_mag(m) * 2^b for m = 0..3 (x) and
// m = 4..7 (y).  P1 §4: FP4 -> FP8 is exact while b stays in the window where
// every such product is an E4M3 value, b in [-8, 6]; outside it the entry is 0
// (the prepack step rejects such scales).
__device__ __forceinline__ uint2 dequant_lut_entry(int s)
{
    int b = s - 127;
    uint32_t lo = 0, hi = 0;
    if (b >= -8 && b <= 6) {
        for (int m = 0; m < 4; m++) {
            lo |= e4m3_rne_sat(ldexpf(e2m1_mag(m), b)) << (8 * m);
            hi |= e4m3_rne_sat(ldexpf(e2m1_mag(m + 4), b)) << (8 * m);
        }
    }
    return make_uint2(lo, hi);
}

// One 16-byte packed FP4 slot (32 codes) -> 32 E4M3 bytes in element order.
// Byte j of the slot holds element 8*(j/4)+j%4 (low nibble) and that +4 (high
// nibble), so per 32-bit word: the low nibbles give elements 8d..8d+3, the
// high nibbles 8d+4..8d+7.  Each magnitude (3 bits) selects a byte of the
// 8-byte table with v_perm_b32; the sign bit is moved to bit 7.  Negative
// zero is kept (0x8 -> 0x80).
__device__ __forceinline__ uint32_t dq_lo(uint32_t w, uint2 L)
{
    return __builtin_amdgcn_perm(L.y, L.x, w & 0x07070707u) | ((w << 4) & 0x80808080u);
}
__device__ __forceinline__ uint32_t dq_hi(uint32_t w, uint2 L)
{
    return __builtin_amdgcn_perm(L.y, L.x, (w >> 4) & 0x07070707u) | (w & 0x80808080u);
}
__device__ __forceinline__ v8i dequant_slot(uint4 w, uint2 L)
{
    v8i o;
    o[0] = (int)dq_lo(w.x, L); o[1] = (int)dq_hi(w.x, L);
    o[2] = (int)dq_lo(w.y, L); o[3] = (int)dq_hi(w.y, L);
    o[4] = (int)dq_lo(w.z, L); o[5] = (int)dq_hi(w.z, L);
    o[6] = (int)dq_lo(w.w, L); o[7] = (int)dq_hi(w.w, L);
    return o;
}

// 16x16 output tile over one 128-wide K chunk on the FP8 matrix cores
// (v_mfma_f32_16x16x128_f8f6f4, both operands E4M3, no block scale).
// Operand lane layout used throughout: lane l holds row/column l%16 and the
// 32 consecutive K elements (l/16)*32 .. +31 of the chunk, as 8 dwords in
// element order.  Result: lane l holds rows 4*(l/16)+i, i = 0..3, column l%16.
__device__ __forceinline__ v4f mfma_chunk(v8i a, v8i b)
{
    v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
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
