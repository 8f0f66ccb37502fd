/*
 * v4moe_oracle.c -- plain, slow CPU oracle of the DeepSeek-V4-style MoE layer
 * forward (route -> dispatch -> linear1 -> SwiGLU -> linear2 -> combine).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or calls
 * this file: it exists so that tests, the smoke check and the CPU baseline of
 * the benchmark can compare the HIP library against an independent reading of
 * the method.  It shares no code, header, table or constant with the HIP path.
 *
 * Sources (the pages; cited by short tag and section):
 *   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
 *        (itsolotime.com/archives/32374)
 *   P2 = "DeepSeek V4架构学习笔记" (67808.cn/a/484462.html)
 *   P4 = "DeepSeek-V4 的暗线之二：训练一台不会失控的万亿参数机器"
 *        (blog.xieydd.top/deepseek-v4-control-part2)
 * and, for the number formats the pages name but do not define, the OCP
 * Microscaling (MX) v1.0 and OCP 8-bit floating point (OFP8) specifications.
 *
 * Precision policy: every quantity the method keeps in fp32 is rounded to
 * fp32 here exactly where the method rounds it; everything in between is done
 * in fp64 or exact integer arithmetic.  Compile with -ffp-contract=off.
 *
 * Pins (tests under tests/ check each function against something other than
 * itself): formats against exhaustive enumeration and torch's casts; top-k
 * against brute force; logits against an exact-rational error bound and
 * closed forms that fix the summation order (one h-ascending chain); the
 * permutation against a stable library sort; the FFN against a closed form
 * and against a dense matmul formulation.  No function here is parity-unpinned.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define EXPORT __attribute__((visibility("default")))

/* Threads the OpenMP loops below use (1 without OpenMP). */
EXPORT int orc_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------------------------------ */
/* Number formats                                                            */
/* ------------------------------------------------------------------------ */

/* FP4 E2M1 (OCP MX v1.0): 1 sign bit, 2 exponent bits (bias 1), 1 mantissa
 * bit; magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.  P1 §4 names MXFP4 for the MoE
 * expert weights. */
EXPORT double orc_e2m1_value(int code)
{
    int e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -mag : mag;
}

/* FP8 E4M3 (OCP OFP8 "E4M3FN"): bias 7, no infinities, S.1111.111 is NaN,
 * largest finite 448, subnormals m*2^-9. */
EXPORT double orc_e4m3_value(int byte)
{
    int e = (byte >> 3) & 15, m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (byte & 0x80) ? -mag : mag;
}

/* Round a real value to E4M3: nearest representable value, ties to the even
 * mantissa, magnitudes beyond the largest finite value saturate to +-448
 * (never NaN).  v must not be NaN. */
EXPORT int orc_e4m3_encode(double v)
{
    int sign = signbit(v) ? 0x80 : 0;
    double a = fabs(v);
    int q, ex;
    if (a >= 464.0)            /* half an ulp above 448 and beyond: saturate */
        return sign | 0x7E;
    if (a < 0x1p-6) {          /* subnormal range: grid step 2^-9 */
        q = (int)nearbyint(a * 512.0);       /* 0..8; 8 is the smallest normal */
        return sign | q;
    }
    frexp(a, &ex);             /* a = f * 2^ex, f in [0.5, 1) */
    ex -= 1;                   /* a = (1 + m/8) * 2^ex, ex in [-6, 8] */
    q = (int)nearbyint(ldexp(a, -ex) * 8.0 - 8.0);
    if (q == 8) { q = 0; ex += 1; }
    q = ((ex + 7) << 3) | q;
    if (q > 0x7E) q = 0x7E;
    return sign | q;
}

/* Value of a 32-bit float pattern read as an unbounded binary float (an all-ones
 * exponent is read as 2^128, not infinity), so that rounding up past the
 * largest finite value compares correctly. */
static double f32_pattern_value(uint32_t u)
{
    int e = (int)((u >> 23) & 0xFF);
    double m = (double)(u & 0x7FFFFF);
    double mag = (e == 0) ? ldexp(m, -149) : ldexp(1.0 + ldexp(m, -23), e - 127);
    return (u >> 31) ? -mag : mag;
}

/* bf16 of a finite fp32 value: of the two bf16 values bracketing f, the
 * nearer one; on a tie, the one with an even last mantissa bit. */
EXPORT uint16_t orc_bf16_encode(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t lo = u & 0xFFFF0000u, hi = lo + 0x10000u;
    double v = (double)f;
    double dlo = fabs(v - f32_pattern_value(lo)), dhi = fabs(f32_pattern_value(hi) - v);
    if (dlo < dhi) return (uint16_t)(lo >> 16);
    if (dhi < dlo) return (uint16_t)(hi >> 16);
    return ((lo >> 16) & 1) ? (uint16_t)(hi >> 16) : (uint16_t)(lo >> 16);
}

EXPORT float orc_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Array forms of the two encoders (used by the format tests). */
EXPORT void orc_e4m3_encode_array(int64_t n, const double* v, uint8_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = (uint8_t)orc_e4m3_encode(v[i]);
}

EXPORT void orc_bf16_encode_array(int64_t n, const float* v, uint16_t* out)
{
    for (int64_t i = 0; i < n; i++) out[i] = orc_bf16_encode(v[i]);
}

/* ------------------------------------------------------------------------ */
/* FP4 -> FP8 dequantisation (P1 §4; P4 §4 "FP4 QAT")                        */
/* ------------------------------------------------------------------------ */

/* The E4M3 byte holding e2m1(code) * 2^b, for sub-block exponent b.  The pages
 * state that this conversion is lossless because E4M3 has two more exponent
 * bits than E2M1, provided the sub-block scales of a 128x128 block stay within
 * a bounded ratio.  Here it is simply "encode the exact product"; whether the
 * result is exact is checked by the tests, not assumed. */
EXPORT int orc_dequant_code(int code, int b)
{
    return orc_e4m3_encode(ldexp(orc_e2m1_value(code), b));
}

/* The same map written as a bit formula, valid where no product falls below
 * the E4M3 normal range (b in [-5, 6]): zero keeps its sign, the E2M1
 * subnormal 0.5 becomes an E4M3 power of two, normal codes add b+6 to the
 * exponent field and keep the mantissa bit. */
EXPORT int orc_dequant_bitmap(int code, int b)
{
    int s = (code & 8) << 4, m = code & 7;
    if (m == 0) return s;
    if (m == 1) return s | ((b + 6) << 3);
    return s | ((m << 2) + ((b + 6) << 3));
}

/* Dequantise one canonical matrix: fp4 [N][K/2] (low nibble = even k),
 * e8m0 [N][K/32] (byte = 127 + b)  ->  E4M3 bytes [N][K]. */
EXPORT void orc_dequant_matrix(int N, int K, const uint8_t* fp4, const uint8_t* e8m0, uint8_t* out)
{
    /* memoised orc_dequant_code: one entry per (code, e8m0 byte) */
    uint8_t lut[16][256];
    for (int c = 0; c < 16; c++)
        for (int s = 0; s < 256; s++)
            lut[c][s] = (uint8_t)orc_dequant_code(c, s - 127);
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++) {
            uint8_t byte = fp4[(size_t)n * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            out[(size_t)n * K + k] = lut[code][e8m0[(size_t)n * (K / 32) + k / 32]];
        }
}

/* ------------------------------------------------------------------------ */
/* Routing (P2 DeepSeekMoE notes: sqrt(softplus) affinity, hash routing)     */
/* ------------------------------------------------------------------------ */

/* Router logits z[t][e] = sum_h x[t][h] * W_r[h][e] (+ bias[e]) (P2,
 * DeepSeekMoE notes: the affinity is taken of this logit).  Reading of the
 * unstated precision and order: one fp32 fused multiply-add per h, h
 * ascending, starting from +0; the bias is one fp32 add afterwards. */
EXPORT void orc_router_logits(int T, int H, int E, const uint16_t* x, const float* wr,
                              const float* bias, float* z)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        float* zt = z + (size_t)t * E;
        for (int e = 0; e < E; e++) zt[e] = 0.0f;
        /* h outer, e inner: each z[t][e] is still its own h-ascending chain */
        for (int h = 0; h < H; h++) {
            float xv = orc_bf16_value(x[(size_t)t * H + h]);
            const float* w = wr + (size_t)h * E;
            for (int e = 0; e < E; e++) zt[e] = fmaf(xv, w[e], zt[e]);
        }
        if (bias)
            for (int e = 0; e < E; e++) zt[e] = zt[e] + bias[e];
    }
}

/* splitmix64 output function (Steele, Lea & Flood, OOPSLA 2014). */
EXPORT uint64_t orc_splitmix64(uint64_t v)
{
    uint64_t z = v + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* Top-k selection and gate weights for every token.
 * mode 0 (learned): repeatedly take the largest remaining logit, the lower
 *   expert id winning ties; slot j holds the j-th pick.  Affinity
 *   a = sqrt(softplus(z)) is computed in fp64 and rounded to fp32; the weights
 *   are normalised over the k picks: w_j = fp32(a_j / sum_i a_i).
 * mode 1 (hash): expert_j = splitmix64(token_id*k + j) mod E, stepping +1 mod
 *   E past experts already picked for this token; w_j = 1/k.
 * token_ids may be NULL (then token_id = t). */
EXPORT void orc_route(int T, int H, int E, int k, const uint16_t* x, const float* wr,
                      const float* bias, int mode, const int64_t* token_ids,
                      int32_t* ids, float* w)
{
    if (mode == 1) {
        for (int t = 0; t < T; t++) {
            uint64_t tid = token_ids ? (uint64_t)token_ids[t] : (uint64_t)t;
            for (int j = 0; j < k; j++) {
                int c = (int)(orc_splitmix64(tid * (uint64_t)k + (uint64_t)j) % (uint64_t)E);
                for (;;) {
                    int dup = 0;
                    for (int i = 0; i < j; i++) dup |= (ids[(size_t)t * k + i] == c);
                    if (!dup) break;
                    c = (c + 1) % E;
                }
                ids[(size_t)t * k + j] = c;
                w[(size_t)t * k + j] = 1.0f / (float)k;
            }
        }
        return;
    }
    float* z = (float*)malloc((size_t)T * E * sizeof(float));
    orc_router_logits(T, H, E, x, wr, bias, z);
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        const float* zt = z + (size_t)t * E;
        char* taken = (char*)calloc((size_t)E, 1);
        float a[64];   /* k <= 64 */
        double sum = 0.0;
        for (int j = 0; j < k; j++) {
            int best = -1;
            for (int e = 0; e < E; e++) {
                if (taken[e]) continue;
                if (best < 0 || zt[e] > zt[best]) best = e;   /* strict: lower id keeps ties */
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
            double zz = (double)zt[best];
            double sp = fmax(zz, 0.0) + log1p(exp(-fabs(zz)));
            a[j] = (float)sqrt(sp);
            sum += (double)a[j];
        }
        for (int j = 0; j < k; j++)
            w[(size_t)t * k + j] = (sum > 0.0) ? (float)((double)a[j] / sum) : 1.0f / (float)k;
        free(taken);
    }
    free(z);
}

/* ------------------------------------------------------------------------ */
/* Activation quantisation: the FP8 dispatch payload (P1 §1.4)               */
/* ------------------------------------------------------------------------ */

/* Per row and per group of 128 consecutive channels: s = fp32(amax / 448)
 * (s = 1 when the group is all zero), q = E4M3(fp32(v / s)).  v is [R][C]. */
EXPORT void orc_quant_rows(int R, int C, const float* v, uint8_t* q, float* s)
{
    int G = C / 128;
    for (int r = 0; r < R; r++)
        for (int g = 0; g < G; g++) {
            const float* vg = v + (size_t)r * C + (size_t)g * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; i++) amax = fmaxf(amax, fabsf(vg[i]));
            float sc = (amax > 0.0f) ? amax / 448.0f : 1.0f;
            s[(size_t)r * G + g] = sc;
            for (int i = 0; i < 128; i++) {
                float y = vg[i] / sc;
                q[(size_t)r * C + (size_t)g * 128 + i] = (uint8_t)orc_e4m3_encode((double)y);
            }
        }
}

/* x (bf16 bits [T][H]) -> xq (E4M3 [T][H]) and xs (fp32 [T][H/128]). */
EXPORT void orc_quant_x(int T, int H, const uint16_t* x, uint8_t* xq, float* xs)
{
#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        float* row = (float*)malloc((size_t)H * sizeof(float));
        for (int h = 0; h < H; h++) row[h] = orc_bf16_value(x[(size_t)t * H + h]);
        orc_quant_rows(1, H, row, xq + (size_t)t * H, xs + (size_t)t * (H / 128));
        free(row);
    }
}

/* ------------------------------------------------------------------------ */
/* Weight quantisation: FP32 master weights -> MXFP4 under 128x128 blocks      */
/* (P1 §4, P4 §4: the QAT forward quantises the FP32 master weights to MXFP4;  */
/* the pages cite the OCP MX paper for the format and give no formulas, so the */
/* readings are stated here).                                                  */
/* ------------------------------------------------------------------------ */

/* Nearest E2M1 code of x: ties go to the even code (mantissa bit 0),
 * magnitudes at or beyond 6 saturate to 6, the sign of x is kept (also when
 * the magnitude rounds to zero). */
EXPORT int orc_e2m1_encode(double x)
{
    static const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const int neg = signbit(x) ? 8 : 0;
    const double m = fabs(x);
    int best = 7;
    for (int i = 0; i < 7; i++) {
        const double mid = 0.5 * (grid[i] + grid[i + 1]);
        if (m < mid) { best = i; break; }
        if (m == mid) { best = (i % 2 == 0) ? i : i + 1; break; }
    }
    return neg | best;
}

/* w: fp32 [E][N][K] (N, K multiples of 128) -> canonical fp4 [E][N][K/2],
 * e8m0 [E][N][K/32], blk [E][N/128][K/128].  Per 128x128 block:
 *   s = amax / 384 in fp32 (s = 1 for an all-zero block): the block's largest
 *       magnitude lands on 6 * 2^6, the largest value an FP4 element reaches
 *       at the top of the lossless window b <= 6 (and 384 <= 448, E4M3's max);
 *   per 1x32 sub-block of a row: v = w / s in fp32; b = floor(log2(max|v|))
 *       - 2 (the OCP MX shared-exponent rule, E2M1's largest exponent being
 *       2), raised to -8 when below the window (the sub-block is then counted
 *       as clamped: its scale ratio to the block exceeds what E4M3 absorbs),
 *       b = 0 for an all-zero sub-block; codes = orc_e2m1_encode(v * 2^-b).
 * Returns the number of clamped sub-blocks. */
EXPORT int64_t orc_quantize_weights(int E, int N, int K, const float* w, uint8_t* fp4, uint8_t* e8m0,
                                    float* blk)
{
    const int NB = N / 128, KB = K / 128;
    int64_t clamped = 0;
#pragma omp parallel for schedule(dynamic) reduction(+ : clamped)
    for (long id = 0; id < (long)E * NB * KB; id++) {
        const int e = (int)(id / ((long)NB * KB)), nb = (int)((id / KB) % NB), kb = (int)(id % KB);
        const float* src = w + ((size_t)e * N + (size_t)nb * 128) * K + (size_t)kb * 128;
        float amax = 0.0f;
        for (int r = 0; r < 128; r++)
            for (int c = 0; c < 128; c++) {
                const float a = fabsf(src[(size_t)r * K + c]);
                if (a > amax) amax = a;
            }
        const float s = amax > 0.0f ? amax / 384.0f : 1.0f;
        blk[((size_t)e * NB + nb) * KB + kb] = s;
        for (int r = 0; r < 128; r++) {
            const size_t n = (size_t)e * N + (size_t)nb * 128 + r;
            for (int sb = 0; sb < 4; sb++) {
                float v[32];
                float am = 0.0f;
                for (int j = 0; j < 32; j++) {
                    v[j] = src[(size_t)r * K + sb * 32 + j] / s;
                    if (fabsf(v[j]) > am) am = fabsf(v[j]);
                }
                int b = 0;
                if (am > 0.0f) {
                    int ex;
                    frexp((double)am, &ex);   /* am = m * 2^ex, m in [0.5, 1) */
                    b = (ex - 1) - 2;
                    if (b < -8) { b = -8; clamped++; }
                    if (b > 6) b = 6;
                }
                e8m0[n * (K / 32) + (size_t)kb * 4 + sb] = (uint8_t)(127 + b);
                for (int j = 0; j < 32; j += 2) {
                    const int lo = orc_e2m1_encode(ldexp((double)v[j], -b));
                    const int hi = orc_e2m1_encode(ldexp((double)v[j + 1], -b));
                    fp4[n * (K / 2) + ((size_t)kb * 128 + sb * 32 + j) / 2] = (uint8_t)(lo | (hi << 4));
                }
            }
        }
    }
    return clamped;
}

/* ------------------------------------------------------------------------ */
/* Dispatch as a local permutation (P1 §1.1-§1.2; token order, P1 §3.2)      */
/* ------------------------------------------------------------------------ */

/* Stable counting sort of the pair ids p = t*k + j by expert id.
 * offsets[E+1] is the exclusive scan of the per-expert counts;
 * sorted_pair[pos] = p and pair_pos[p] = pos. */
EXPORT void orc_permute(int T, int k, int E, const int32_t* ids, int32_t* offsets,
                        int32_t* sorted_pair, int32_t* pair_pos)
{
    int P = T * k;
    int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int e = 0; e <= E; e++) offsets[e] = 0;
    for (int p = 0; p < P; p++) offsets[ids[p] + 1] += 1;
    for (int e = 0; e < E; e++) offsets[e + 1] += offsets[e];
    for (int p = 0; p < P; p++) {
        int e = ids[p];
        int pos = offsets[e] + seen[e]++;
        sorted_pair[pos] = p;
        pair_pos[p] = pos;
    }
    free(seen);
}

/* ------------------------------------------------------------------------ */
/* Expert FFN (P1 §1.4: SwiGLU gate/up/down; P1 §4: FP4 weights used as FP8) */
/* ------------------------------------------------------------------------ */

typedef struct {
    const uint8_t* fp4[3];   /* gate, up: [E][I][H/2]; down: [E][H][I/2] */
    const uint8_t* e8m0[3];  /* gate, up: [E][I][H/32]; down: [E][H][I/32] */
    const float* blk[3];     /* gate, up: [E][I/128][H/128]; down: [E][H/128][I/128] */
} orc_weights;

/* One expert matrix as exact integers: W_int = value(E4M3 byte) * 2^9. */
typedef struct {
    int N, K;
    int32_t* wint;           /* [N][K] */
    const float* blk;        /* [N/128][K/128] */
} int_matrix;

static int32_t e4m3_int(int byte)   /* value * 2^9, exact for every finite E4M3 */
{
    return (int32_t)ldexp(orc_e4m3_value(byte), 9);
}

static void make_int_matrix(int_matrix* m, int N, int K, const uint8_t* fp4,
                            const uint8_t* e8m0, const float* blk)
{
    /* memoised dequantisation: one table entry per (code, e8m0 byte) */
    int32_t lut[16][256];
    for (int c = 0; c < 16; c++)
        for (int s = 0; s < 256; s++) {
            int b = s - 127;
            lut[c][s] = (b >= -30 && b <= 30) ? e4m3_int(orc_dequant_code(c, b)) : 0;
        }
    m->N = N;
    m->K = K;
    m->blk = blk;
    m->wint = (int32_t*)malloc((size_t)N * K * sizeof(int32_t));
#pragma omp parallel for schedule(static)
    for (int n = 0; n < N; n++)
        for (int k = 0; k < K; k++) {
            uint8_t byte = fp4[(size_t)n * (K / 2) + k / 2];
            int code = (k & 1) ? (byte >> 4) : (byte & 15);
            m->wint[(size_t)n * K + k] = lut[code][e8m0[(size_t)n * (K / 32) + k / 32]];
        }
}

/* y[n] = sum over 128-wide K chunks c of  s_in[c] * blk[n/128][c] * P_c,
 * where P_c = sum_{k in c} value(in_q[k]) * value(W[n][k]) is computed exactly
 * (as an integer scaled by 2^-18) and the chunk terms are summed in fp64. */
static void expert_linear(const int_matrix* m, const int32_t* xint, const float* s_in, double* y)
{
    int N = m->N, K = m->K, C = K / 128;
    for (int n = 0; n < N; n++) {
        const int32_t* wr = m->wint + (size_t)n * K;
        double acc = 0.0;
        for (int c = 0; c < C; c++) {
            int64_t P = 0;
            for (int i = c * 128; i < c * 128 + 128; i++) P += (int64_t)xint[i] * (int64_t)wr[i];
            acc += (double)s_in[c] * (double)m->blk[(size_t)(n / 128) * C + c] * ldexp((double)P, -18);
        }
        y[n] = acc;
    }
}

/* The activation between the two expert matmuls.
 *   ORC_ACT_SWIGLU: h = SiLU(G) * U, SiLU(g) = g / (1 + exp(-g)) (P1 §1.4);
 *   ORC_ACT_RELU2, ORC_ACT_RELU: the gate-less FFN the pages propose as the
 *   cheap alternative (P1, the hardware suggestions closing §1: an elementwise
 *   activation needing neither exponential nor division, and no gate
 *   projection so that the intermediate can be wider at the same parameter
 *   count): h = max(U, 0)^2 or h = max(U, 0).  The pages name no function;
 *   squared ReLU and ReLU are the two taken here. */
#define ORC_ACT_SWIGLU 0
#define ORC_ACT_RELU2  1
#define ORC_ACT_RELU   2

static float activation(int act, double G, double U)
{
    switch (act) {
    case ORC_ACT_RELU2: { const double r = U > 0.0 ? U : 0.0; return (float)(r * r); }
    case ORC_ACT_RELU: return (float)(U > 0.0 ? U : 0.0);
    default: return (float)(G / (1.0 + exp(-G)) * U);
    }
}

/* One (token, expert) pair: x row already quantised (xq, xs).
 * G, U rounded to fp32; h = fp32(activation(G, U)) (mg unused by the
 * gate-less activations); h quantised per 128 channels like x; Y = down(h) in
 * fp64, then either bf16(fp32(Y)) (normal mode) or kept in fp64 (exact mode,
 * y_exact != NULL). */
static void pair_ffn(int act, int H, int I, const int_matrix* mg, const int_matrix* mu, const int_matrix* md,
                     const uint8_t* xq, const float* xs, uint16_t* y_bf16, double* y_exact,
                     double* G_out, double* U_out, uint8_t* hq_out, float* hs_out)
{
    int32_t* xint = (int32_t*)malloc((size_t)H * sizeof(int32_t));
    double* g = (double*)malloc((size_t)I * sizeof(double));
    double* u = (double*)malloc((size_t)I * sizeof(double));
    float* h = (float*)malloc((size_t)I * sizeof(float));
    uint8_t* hq = (uint8_t*)malloc((size_t)I);
    float* hs = (float*)malloc((size_t)(I / 128) * sizeof(float));
    int32_t* hint = (int32_t*)malloc((size_t)I * sizeof(int32_t));
    double* y = (double*)malloc((size_t)H * sizeof(double));

    for (int i = 0; i < H; i++) xint[i] = e4m3_int(xq[i]);
    if (act == ORC_ACT_SWIGLU) expert_linear(mg, xint, xs, g);
    expert_linear(mu, xint, xs, u);
    for (int n = 0; n < I; n++) {
        double G = act == ORC_ACT_SWIGLU ? (double)(float)g[n] : 0.0, U = (double)(float)u[n];
        h[n] = activation(act, G, U);
        if (G_out) G_out[n] = G;
        if (U_out) U_out[n] = U;
    }
    orc_quant_rows(1, I, h, hq, hs);
    if (hq_out) memcpy(hq_out, hq, (size_t)I);
    if (hs_out) memcpy(hs_out, hs, (size_t)(I / 128) * sizeof(float));
    for (int n = 0; n < I; n++) hint[n] = e4m3_int(hq[n]);
    expert_linear(md, hint, hs, y);
    for (int n = 0; n < H; n++) {
        if (y_exact) y_exact[n] = y[n];
        if (y_bf16) y_bf16[n] = orc_bf16_encode((float)y[n]);
    }
    free(xint); free(g); free(u); free(h); free(hq); free(hs); free(hint); free(y);
}

/* ------------------------------------------------------------------------ */
/* Whole layer                                                               */
/* ------------------------------------------------------------------------ */

/* Forward of the MoE layer for all T tokens, or -- when subset != NULL -- the
 * expert FFN and combine only for the tokens listed in subset[0..n_subset)
 * (routing, quantisation and the permutation always cover all T tokens).
 *
 * Outputs (any may be NULL except where noted):
 *   ids, w         [T][k]            routing (required)
 *   offsets        [E+1], sorted_pair / pair_pos [T*k]  (required)
 *   xq [T][H], xs [T][H/128]          quantised dispatch payload (required)
 *   y   [T*k][H] bf16 bits            expert outputs in pair order p = t*k+j
 *   out [T][H]   bf16 bits            out[t] = bf16(fp32(sum_j w_j * Y[t*k+j]))
 *   out_exact [T][H] fp64            exact mode: no rounding of Y or out
 * act selects the activation (ORC_ACT_*); the gate-less ones never read the
 * gate matrix.  Rows of y/out/out_exact that belong to tokens outside the
 * subset are left untouched.  Returns 0. */
EXPORT int orc_layer_forward(int T, int H, int I, int E, int k, int act,
                             const uint16_t* x, const float* wr, const float* bias,
                             int mode, const int64_t* token_ids, const orc_weights* W,
                             int32_t* ids, float* w, int32_t* offsets, int32_t* sorted_pair,
                             int32_t* pair_pos, uint8_t* xq, float* xs,
                             uint16_t* y, uint16_t* out, double* out_exact,
                             const int32_t* subset, int n_subset)
{
    int P = T * k;
    orc_route(T, H, E, k, x, wr, bias, mode, token_ids, ids, w);
    orc_quant_x(T, H, x, xq, xs);
    orc_permute(T, k, E, ids, offsets, sorted_pair, pair_pos);

    char* want = (char*)calloc((size_t)(T > 0 ? T : 1), 1);
    if (subset) {
        for (int i = 0; i < n_subset; i++) want[subset[i]] = 1;
    } else {
        memset(want, 1, (size_t)T);
    }
    uint16_t* ybuf = (uint16_t*)malloc((size_t)(P > 0 ? P : 1) * H * sizeof(uint16_t));
    double* yex = out_exact ? (double*)malloc((size_t)(P > 0 ? P : 1) * H * sizeof(double)) : NULL;

    /* Experts with at least one wanted row.  Every pair's result depends only
     * on its own token and expert, so the order in which experts and pairs
     * are visited changes nothing: with fewer wanted pairs per expert than
     * threads the experts are spread over the threads (one at a time per
     * thread), otherwise the pairs of one expert are. */
    int* todo = (int*)malloc((size_t)E * sizeof(int));
    int ntodo = 0, npairs = 0;
    for (int e = 0; e < E; e++) {
        int need = 0;
        for (int r = offsets[e]; r < offsets[e + 1]; r++) need += want[sorted_pair[r] / k];
        if (need) todo[ntodo++] = e;
        npairs += need;
    }
    const int by_expert = ntodo > 1 && npairs < ntodo * orc_num_threads();
#pragma omp parallel for schedule(dynamic, 1) if (by_expert)
    for (int i = 0; i < ntodo; i++) {
        const int e = todo[i];
        int lo = offsets[e], hi = offsets[e + 1];
        int_matrix mg = {0}, mu, md;
        size_t so = (size_t)e;
        if (act == ORC_ACT_SWIGLU)
            make_int_matrix(&mg, I, H, W->fp4[0] + so * I * (H / 2), W->e8m0[0] + so * I * (H / 32),
                            W->blk[0] + so * (I / 128) * (H / 128));
        make_int_matrix(&mu, I, H, W->fp4[1] + so * I * (H / 2), W->e8m0[1] + so * I * (H / 32),
                        W->blk[1] + so * (I / 128) * (H / 128));
        make_int_matrix(&md, H, I, W->fp4[2] + so * H * (I / 2), W->e8m0[2] + so * H * (I / 32),
                        W->blk[2] + so * (H / 128) * (I / 128));
#pragma omp parallel for schedule(dynamic, 1) if (!by_expert)
        for (int r = lo; r < hi; r++) {
            int p = sorted_pair[r], t = p / k;
            if (!want[t]) continue;
            pair_ffn(act, H, I, &mg, &mu, &md, xq + (size_t)t * H, xs + (size_t)t * (H / 128),
                     ybuf + (size_t)p * H, yex ? yex + (size_t)p * H : NULL, NULL, NULL, NULL, NULL);
        }
        free(mg.wint); free(mu.wint); free(md.wint);
    }
    free(todo);

#pragma omp parallel for schedule(static)
    for (int t = 0; t < T; t++) {
        if (!want[t]) continue;
        for (int n = 0; n < H; n++) {
            double acc = 0.0, acc_ex = 0.0;
            for (int j = 0; j < k; j++) {
                size_t p = (size_t)t * k + j;
                acc += (double)w[p] * (double)orc_bf16_value(ybuf[p * H + n]);
                if (yex) acc_ex += (double)w[p] * yex[p * H + n];
            }
            if (out) out[(size_t)t * H + n] = orc_bf16_encode((float)acc);
            if (out_exact) out_exact[(size_t)t * H + n] = acc_ex;
        }
        if (y)
            for (int j = 0; j < k; j++) {
                size_t p = (size_t)t * k + j;
                memcpy(y + p * H, ybuf + p * H, (size_t)H * sizeof(uint16_t));
            }
    }
    free(want);
    free(ybuf);
    free(yex);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward of the layer                                                     */
/* (P1 §3 and P4 §3: the MoE backward accumulates in a fixed, token-ordered   */
/* sequence, no atomics; P1 §4 and P4 §4: gradients are computed with the     */
/* forward's FP8 weights and passed straight to the FP32 master weights, i.e. */
/* the straight-through estimator for every quantisation step, and the        */
/* transposed weights are the same FP8 values, never requantised.)            */
/* ------------------------------------------------------------------------ */

/* Real value of weight (n, k) of an expert matrix: E4M3 value x block scale. */
static double wreal(const int_matrix* m, int n, int k)
{
    return ldexp((double)m->wint[(size_t)n * m->K + k], -9) *
           (double)m->blk[(size_t)(n / 128) * (m->K / 128) + k / 128];
}

/* Derivatives of the activations at (G, U): dh/dG and dh/dU. */
static void activation_grad(int act, double G, double U, double* dG, double* dU)
{
    switch (act) {
    case ORC_ACT_RELU2: *dG = 0.0; *dU = U > 0.0 ? 2.0 * U : 0.0; return;
    case ORC_ACT_RELU: *dG = 0.0; *dU = U > 0.0 ? 1.0 : 0.0; return;
    default: {
        const double sg = 1.0 / (1.0 + exp(-G));          /* sigmoid */
        *dG = U * sg * (1.0 + G * (1.0 - sg));            /* d/dG [G sigmoid(G) U] */
        *dU = G * sg;                                     /* SiLU(G) */
    }
    }
}

/* Gradients of L = sum(dout * out) for the layer forward above, in fp64.
 * The forward is recomputed exactly as orc_layer_forward does it; then, per
 * (token, expert) pair p = t*k + j of expert e with routing weight w_p:
 *   dY_p = w_p * dout_t                        (out = sum_j w_j Y_j)
 *   dw_p = <dout_t, Y_p>, Y_p the bf16 expert output the combine used
 *   dh_p = Wd_e^T dY_p                         (real FP8 weight values)
 *   dG_p, dU_p = dh_p * dh/dG, dh_p * dh/dU at the forward's fp32 G, U
 *   dx_p = Wg_e^T dG_p + Wu_e^T dU_p,   dx_t = sum over j ascending of dx_{t,j}
 *   dWd_e = sum_p dY_p hq_p^T,  dWg_e = sum_p dG_p xq_p^T,  dWu_e = sum_p dU_p xq_p^T
 * where xq_p, hq_p are the forward's quantised activations (E4M3 value x fp32
 * scale) and the sums over p run over the expert's rows in their sorted
 * (token) order.  The quantisations are straight-through: their gradient is
 * the identity, so dx and the dW's are the gradients with respect to x and to
 * the FP32 master weights.  The router is not differentiated (dw is returned
 * for it).  For the gate-less activations the gate terms vanish.
 * Outputs (each may be NULL): dx [T][H], dw [T][k], dWg, dWu [E][I][H],
 * dWd [E][H][I].  tok / n_tok restrict dx and dw to the listed tokens (their
 * rows are written; others are left untouched); ex / n_ex restrict the dW's to
 * the listed experts, whose gradients are then stored in the order of the list
 * (dWg [n_ex][I][H] ...).  Returns 0. */
EXPORT int orc_layer_backward(int T, int H, int I, int E, int k, int act,
                              const uint16_t* x, const float* wr, const float* bias,
                              int mode, const int64_t* token_ids, const orc_weights* W,
                              const uint16_t* dout, double* dx, double* dw,
                              double* dWg, double* dWu, double* dWd,
                              const int32_t* tok, int n_tok, const int32_t* ex, int n_ex)
{
    const int P = T * k;
    int32_t* ids = (int32_t*)malloc((size_t)(P > 0 ? P : 1) * sizeof(int32_t));
    float* w = (float*)malloc((size_t)(P > 0 ? P : 1) * sizeof(float));
    int32_t* offsets = (int32_t*)malloc((size_t)(E + 1) * sizeof(int32_t));
    int32_t* sorted_pair = (int32_t*)malloc((size_t)(P > 0 ? P : 1) * sizeof(int32_t));
    int32_t* pair_pos = (int32_t*)malloc((size_t)(P > 0 ? P : 1) * sizeof(int32_t));
    uint8_t* xq = (uint8_t*)malloc((size_t)(T > 0 ? T : 1) * H);
    float* xs = (float*)malloc((size_t)(T > 0 ? T : 1) * (H / 128) * sizeof(float));
    orc_route(T, H, E, k, x, wr, bias, mode, token_ids, ids, w);
    orc_quant_x(T, H, x, xq, xs);
    orc_permute(T, k, E, ids, offsets, sorted_pair, pair_pos);

    char* want_t = (char*)calloc((size_t)(T > 0 ? T : 1), 1);
    char* want_e = (char*)calloc((size_t)E, 1);
    int* slot_e = (int*)malloc((size_t)E * sizeof(int));        /* output slot of each wanted expert */
    if (tok) { for (int i = 0; i < n_tok; i++) want_t[tok[i]] = 1; } else memset(want_t, 1, (size_t)T);
    for (int e = 0; e < E; e++) slot_e[e] = e;
    if (ex) { for (int i = 0; i < n_ex; i++) { want_e[ex[i]] = 1; slot_e[ex[i]] = i; } }
    else memset(want_e, 1, (size_t)E);
    double* dxp = (double*)calloc((size_t)(P > 0 ? P : 1) * H, sizeof(double));   /* dx per pair */

    for (int e = 0; e < E; e++) {
        const int lo = offsets[e], hi = offsets[e + 1], R = hi - lo;
        int need_t = 0;
        for (int r = lo; r < hi; r++) need_t |= want_t[sorted_pair[r] / k];
        const int need_w = want_e[e] && (dWg || dWu || dWd);
        if (!need_t && !need_w) continue;
        int_matrix mg = {0}, mu, md;
        const size_t so = (size_t)e;
        if (act == ORC_ACT_SWIGLU)
            make_int_matrix(&mg, I, H, W->fp4[0] + so * I * (H / 2), W->e8m0[0] + so * I * (H / 32),
                            W->blk[0] + so * (I / 128) * (H / 128));
        make_int_matrix(&mu, I, H, W->fp4[1] + so * I * (H / 2), W->e8m0[1] + so * I * (H / 32),
                        W->blk[1] + so * (I / 128) * (H / 128));
        make_int_matrix(&md, H, I, W->fp4[2] + so * H * (I / 2), W->e8m0[2] + so * H * (I / 32),
                        W->blk[2] + so * (H / 128) * (I / 128));
        /* per row of the expert: dY, dG, dU, and the quantised activations */
        double* dY = (double*)malloc((size_t)(R > 0 ? R : 1) * H * sizeof(double));
        double* dGr = (double*)malloc((size_t)(R > 0 ? R : 1) * I * sizeof(double));
        double* dUr = (double*)malloc((size_t)(R > 0 ? R : 1) * I * sizeof(double));
        double* hr = (double*)malloc((size_t)(R > 0 ? R : 1) * I * sizeof(double));
        char* done = (char*)calloc((size_t)(R > 0 ? R : 1), 1);
#pragma omp parallel for schedule(dynamic, 1)
        for (int r = lo; r < hi; r++) {
            const int p = sorted_pair[r], t = p / k, rr = r - lo;
            if (!need_w && !want_t[t]) continue;
            double* G = (double*)malloc((size_t)I * sizeof(double));
            double* U = (double*)malloc((size_t)I * sizeof(double));
            uint8_t* hq = (uint8_t*)malloc((size_t)I);
            float* hs = (float*)malloc((size_t)(I / 128) * sizeof(float));
            uint16_t* y = (uint16_t*)malloc((size_t)H * sizeof(uint16_t));
            double* dh = (double*)malloc((size_t)I * sizeof(double));
            pair_ffn(act, H, I, &mg, &mu, &md, xq + (size_t)t * H, xs + (size_t)t * (H / 128), y, NULL,
                     G, U, hq, hs);
            double* dYr = dY + (size_t)rr * H;
            double dwp = 0.0;
            for (int n = 0; n < H; n++) {
                const double g = (double)orc_bf16_value(dout[(size_t)t * H + n]);
                dYr[n] = (double)w[p] * g;
                dwp += g * (double)orc_bf16_value(y[n]);
            }
            if (dw && want_t[t]) dw[p] = dwp;
            for (int i = 0; i < I; i++) {
                double a = 0.0;
                for (int n = 0; n < H; n++) a += dYr[n] * wreal(&md, n, i);
                dh[i] = a;
            }
            for (int i = 0; i < I; i++) {
                double gG, gU;
                activation_grad(act, G[i], U[i], &gG, &gU);
                dGr[(size_t)rr * I + i] = dh[i] * gG;
                dUr[(size_t)rr * I + i] = dh[i] * gU;
                hr[(size_t)rr * I + i] = orc_e4m3_value(hq[i]) * (double)hs[i / 128];
            }
            if (want_t[t]) {
                double* d = dxp + (size_t)p * H;
                for (int h = 0; h < H; h++) {
                    double a = 0.0;
                    for (int i = 0; i < I; i++) {
                        if (act == ORC_ACT_SWIGLU) a += dGr[(size_t)rr * I + i] * wreal(&mg, i, h);
                        a += dUr[(size_t)rr * I + i] * wreal(&mu, i, h);
                    }
                    d[h] = a;
                }
            }
            done[rr] = 1;
            free(G); free(U); free(hq); free(hs); free(y); free(dh);
        }
        if (need_w) {
            /* weight gradients: rows accumulated in sorted order, one output
             * element per iteration (parallel over outputs, never over rows) */
            if (dWd) {
                double* o = dWd + (size_t)slot_e[e] * H * I;
#pragma omp parallel for schedule(static)
                for (int n = 0; n < H; n++)
                    for (int i = 0; i < I; i++) {
                        double a = 0.0;
                        for (int rr = 0; rr < R; rr++) a += dY[(size_t)rr * H + n] * hr[(size_t)rr * I + i];
                        o[(size_t)n * I + i] = a;
                    }
            }
            for (int m = 0; m < 2; m++) {
                double* o = m == 0 ? dWg : dWu;
                const double* d = m == 0 ? dGr : dUr;
                if (!o || (m == 0 && act != ORC_ACT_SWIGLU)) continue;
                o += (size_t)slot_e[e] * I * H;
#pragma omp parallel for schedule(static)
                for (int i = 0; i < I; i++)
                    for (int h = 0; h < H; h++) {
                        double a = 0.0;
                        for (int rr = 0; rr < R; rr++) {
                            const int t = sorted_pair[lo + rr] / k;
                            a += d[(size_t)rr * I + i] * orc_e4m3_value(xq[(size_t)t * H + h]) *
                                 (double)xs[(size_t)t * (H / 128) + h / 128];
                        }
                        o[(size_t)i * H + h] = a;
                    }
            }
        }
        free(dY); free(dGr); free(dUr); free(hr); free(done);
        free(mg.wint); free(mu.wint); free(md.wint);
    }
    if (dx)
#pragma omp parallel for schedule(static)
        for (int t = 0; t < T; t++) {
            if (!want_t[t]) continue;
            for (int h = 0; h < H; h++) {
                double a = 0.0;
                for (int j = 0; j < k; j++) a += dxp[((size_t)t * k + j) * H + h];
                dx[(size_t)t * H + h] = a;
            }
        }
    free(ids); free(w); free(offsets); free(sorted_pair); free(pair_pos); free(xq); free(xs);
    free(want_t); free(want_e); free(slot_e); free(dxp);
    return 0;
}
