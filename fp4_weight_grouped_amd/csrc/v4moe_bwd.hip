// libv4moe -- backward of the MoE layer on gfx950.
//
// Sources (the pages; cited by short tag and section):
//   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
//   P4 = "DeepSeek-V4 的暗线之二：训练一台不会失控的万亿参数机器"
// P1 §3 / P4 §3: the MoE backward must accumulate in a fixed order (the pages
// order tokens before accumulation and isolate buffers instead of racing on
// atomics).  P1 §4 / P4 §4: gradients are computed with the forward's FP8
// weights and passed straight to the FP32 master weights (straight-through
// quantisation), and since FP4 -> FP8 is lossless the transposed weights are
// the same FP8 values, never requantised.
//
// With L = sum(dout * out), per (token t, expert e) pair p = t*k + j of weight
// w_p, in expert-sorted row order r:
//   dY_r  = w_p dout_t                          (k_bwd_combine; also dw_p = <dout_t, Y_p>)
//   dh_r  = Wd_e^T dY_r, then dG_r, dU_r        (k_bgemm<DGRAD2>, activation derivative fused)
//   dx_r  = [Wg_e; Wu_e]^T [dG_r; dU_r]         (k_bgemm<DGRAD1>)
//   dx_t  = sum_j dx_{t,j}, j ascending         (k_bwd_unpermute)
//   dW_e  = sum_r (row gradient) (forward activation)^T over the expert's rows
//           in sorted order                     (k_bwd_transpose + k_bgemm<WGRAD>)
// Every matrix product runs on the bf16 matrix cores (v_mfma_f32_16x16x32_bf16)
// with fp32 accumulation: FP8 weight values, FP8 activation codes and E4M3
// values are exact in bf16; the incoming gradients are rounded to bf16, and
// so are the activations of the weight gradients (E4M3 code times its fp32
// scale).  The weights' 128x128 block scales multiply each 128-wide K chunk's
// partial sum (as in the forward).  No atomics: every output element is
// written once by one thread, in a fixed reduction order.
#include "v4moe_device.h"
#include "v4moe_internal.h"

#include <hip/hip_runtime.h>

namespace v4moe {

namespace {

typedef __bf16 bf8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ uint16_t bf16_bits(float f)
{
    return (uint16_t)bf16x2(f, 0.0f);
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t b)
{
    // E4M3FN: bias 7, subnormals at exponent field 0; never NaN here
    const uint32_t s = (b & 0x80u) << 24, e = (b >> 3) & 15u, m = b & 7u;
    const float mag = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return __uint_as_float(__float_as_uint(mag) | s);
}

}  // namespace

// ---------------------------------------------------------------------------
// Combine backward: dY in sorted row order (bf16) and the routing-weight
// gradients.  One block per pair; the dot product is reduced in a fixed tree.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_combine(int H, int k, const uint16_t* __restrict__ dout,
                                                     const float* __restrict__ w, const uint16_t* __restrict__ y,
                                                     const int32_t* __restrict__ pair_pos,
                                                     uint16_t* __restrict__ dys, float* __restrict__ dw)
{
    __shared__ float red[256];
    const int p = blockIdx.x, t = p / k, tid = threadIdx.x;
    const float wp = w[p];
    const size_t row = (size_t)pair_pos[p];
    float acc = 0.0f;
    for (int n = tid * 8; n < H; n += 2048) {
        const uint4 g = *reinterpret_cast<const uint4*>(dout + (size_t)t * H + n);
        const uint4 yy = *reinterpret_cast<const uint4*>(y + (size_t)p * H + n);
        const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, yw[4] = {yy.x, yy.y, yy.z, yy.w};
        uint32_t o[4];
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const float g0 = __uint_as_float(gw[q] << 16), g1 = __uint_as_float(gw[q] & 0xFFFF0000u);
            const float y0 = __uint_as_float(yw[q] << 16), y1 = __uint_as_float(yw[q] & 0xFFFF0000u);
            acc = __builtin_fmaf(g0, y0, acc);
            acc = __builtin_fmaf(g1, y1, acc);
            o[q] = bf16x2(wp * g0, wp * g1);
        }
        *reinterpret_cast<uint4*>(dys + row * H + n) = make_uint4(o[0], o[1], o[2], o[3]);
    }
    red[tid] = acc;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (tid < s) red[tid] += red[tid + s];
        __syncthreads();
    }
    if (tid == 0) dw[p] = red[0];
}

// ---------------------------------------------------------------------------
// Transposed FP8 weight values as E4M3 bytes: packed matrix (N rows, K
// inputs) -> out[e][kk][nofs + n] = E4M3(e2m1(code) * 2^b) for kk < K, n < N,
// row pitch ldo bytes (so gate and up can share one [H][2I] buffer).  Inside
// the scale window every such value is an E4M3 value, so the bytes are exact;
// a zero keeps its code's sign.  One block per (expert, 64-row quad,
// 128-wide chunk); the quad is transposed through LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_weights_t(int N, int K, const uint8_t* __restrict__ fp4,
                                                   const uint8_t* __restrict__ e8, uint8_t* __restrict__ out,
                                                   int ldo, int nofs, size_t out_expert_stride)
{
    __shared__ uint8_t tr[128][64 + 16];
    const int C = K / 128;
    const int c = blockIdx.x % C;
    const int qd = (blockIdx.x / C) % (N / 64);
    const size_t e = blockIdx.x / ((size_t)C * (N / 64));
    const int tid = threadIdx.x, tq = tid >> 6, sl = tid & 63;
    const int tile = qd * 4 + tq;
    const uint4 codes = *reinterpret_cast<const uint4*>(fp4 + (((e * (N / 16) + tile) * C + c) * 64 + sl) * 16);
    const int b = (int)e8[((e * (N / 64) + qd) * C + c) * 256 + sl * 4 + tq] - 127;
    const uint32_t cw[4] = {codes.x, codes.y, codes.z, codes.w};
    const int nl = tq * 16 + (sl & 15), kl = (sl >> 4) * 32;
#pragma unroll
    for (int i = 0; i < 32; i++) {
        const uint32_t code = (cw[i >> 3] >> (4 * (i & 7))) & 15u;
        const uint32_t e2 = (code >> 1) & 3u, m = code & 1u;
        // e2m1 magnitude as fp32 bits, times 2^b (exact), to its E4M3 byte
        // (exact inside the window), the code's sign bit on top
        const float mag = e2 ? __uint_as_float(((e2 + 126u) << 23) | (m << 22)) : 0.5f * (float)m;
        tr[kl + i][nl] = (uint8_t)((e4m3x2(ldexpf(mag, b), 0.0f) & 0x7Fu) | ((code & 8u) << 4));
    }
    __syncthreads();
    for (int idx = tid; idx < 128 * 4; idx += 256) {
        const int kk = idx >> 2, seg = idx & 3;
        *reinterpret_cast<uint4*>(out + e * out_expert_stride + (size_t)(c * 128 + kk) * ldo + nofs + qd * 64 +
                                  seg * 16) = *reinterpret_cast<const uint4*>(&tr[kk][seg * 16]);
    }
}

// Eight OCP E4M3 bytes -> eight bf16 (exact: every E4M3 value is a bf16
// value), in order: the hardware decode to fp32 (verified here on all 256
// codes), then the upper halves of the fp32 words.
__device__ __forceinline__ uint4 e4m3x8_to_bf16x8(uint2 v)
{
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, false);
    const f2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.x, true);
    const f2 c = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, false);
    const f2 d = __builtin_amdgcn_cvt_pk_f32_fp8((int)v.y, true);
    auto hi2 = [](float lo, float hi) {
        return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
    };
    return make_uint4(hi2(a.x, a.y), hi2(b.x, b.y), hi2(c.x, c.y), hi2(d.x, d.y));
}

// ---------------------------------------------------------------------------
// Padded column offsets of the experts' row segments (multiples of 32) for the
// transposed activation buffers; one block.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void k_pad_offsets(int E, const int32_t* __restrict__ off,
                                                      int32_t* __restrict__ padoff)
{
    __shared__ int s[1024];
    const int tid = threadIdx.x;
    const int cnt = tid < E ? off[tid + 1] - off[tid] : 0;
    s[tid] = (cnt + 31) & ~31;
    __syncthreads();
    for (int d = 1; d < 1024; d <<= 1) {
        const int v = tid >= d ? s[tid - d] : 0;
        __syncthreads();
        s[tid] += v;
        __syncthreads();
    }
    if (tid < E) padoff[tid + 1] = s[tid];
    if (tid == 0) padoff[0] = 0;
}

// ---------------------------------------------------------------------------
// Transpose of sorted-row activations into [channel][padded column] bf16,
// zeros in each expert's padding.  MODE 0: bf16 rows src[r][C] (row pitch
// C); MODE 1: the forward's x payload, E4M3 code x scale of token
// sorted_pair[r]/k; MODE 2: the forward's h payload, hq[r] x hs[r].
// One block per (64 padded columns, 64 channels).
// ---------------------------------------------------------------------------
template <int MODE>
__global__ __launch_bounds__(256) void k_bwd_transpose(int C, int E, int k, const int32_t* __restrict__ off,
                                                       const int32_t* __restrict__ padoff,
                                                       const int32_t* __restrict__ sorted_pair,
                                                       const uint16_t* __restrict__ src16,
                                                       const uint8_t* __restrict__ q8, const float* __restrict__ qs,
                                                       int qs_stride, uint16_t* __restrict__ dst, int ldd)
{
    __shared__ uint16_t tile[64][64 + 2];
    const int pc0 = blockIdx.x * 64, ch0 = blockIdx.y * 64;
    const int total = padoff[E];
    if (pc0 >= total) return;
    const int tid = threadIdx.x;
    // each thread loads 16 channels of one padded column
    {
        const int col = tid >> 2, cseg = (tid & 3) * 16;
        const int pc = pc0 + col;
        int lo = 0, hi = E;                       // expert of pc: padoff[e] <= pc < padoff[e+1]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (padoff[mid] <= pc) lo = mid; else hi = mid;
        }
        const int e = lo;
        const int r = off[e] + (pc - padoff[e]);
        const bool valid = pc < total && r < off[e + 1];
        uint16_t v[16];
        if (!valid) {
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = 0;
        } else if (MODE == 0) {
            const uint4 a = *reinterpret_cast<const uint4*>(src16 + (size_t)r * C + ch0 + cseg);
            const uint4 b = *reinterpret_cast<const uint4*>(src16 + (size_t)r * C + ch0 + cseg + 8);
            const uint32_t wv[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 8; i++) { v[2 * i] = (uint16_t)wv[i]; v[2 * i + 1] = (uint16_t)(wv[i] >> 16); }
        } else {
            const size_t qrow = MODE == 1 ? (size_t)(sorted_pair[r] / k) : (size_t)r;
            const uint4 a = *reinterpret_cast<const uint4*>(q8 + qrow * C + ch0 + cseg);
            const float sc = qs[qrow * qs_stride + (ch0 + cseg) / 128];
            const uint32_t wv[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int i = 0; i < 16; i++) v[i] = bf16_bits(e4m3_to_f32((wv[i >> 2] >> (8 * (i & 3))) & 255u) * sc);
        }
#pragma unroll
        for (int i = 0; i < 16; i++) tile[cseg + i][col] = v[i];
    }
    __syncthreads();
    // write 64 channel rows of 64 columns (128 bytes), 16 bytes per thread
    for (int idx = tid; idx < 64 * 8; idx += 256) {
        const int ch = idx >> 3, seg = idx & 7;
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; i++)
            o[i] = (uint32_t)tile[ch][seg * 8 + 2 * i] | ((uint32_t)tile[ch][seg * 8 + 2 * i + 1] << 16);
        *reinterpret_cast<uint4*>(dst + (size_t)(ch0 + ch) * ldd + pc0 + seg * 8) = make_uint4(o[0], o[1], o[2], o[3]);
    }
}

// ---------------------------------------------------------------------------
// dx_t = sum_j dx_{t,j} in j order (fp32).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_bwd_unpermute(int T, int H, int k, const int32_t* __restrict__ pair_pos,
                                                       const float* __restrict__ dxs, float* __restrict__ dx)
{
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;       // float4 index
    if (idx >= (size_t)T * H / 4) return;
    const size_t t = idx / (H / 4), c = (idx % (H / 4)) * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int j = 0; j < k; j++) {
        const float4 v = *reinterpret_cast<const float4*>(dxs + (size_t)pair_pos[t * k + j] * H + c);
        a.x += v.x; a.y += v.y; a.z += v.z; a.w += v.w;
    }
    *reinterpret_cast<float4*>(dx + t * H + c) = a;
}

// ---------------------------------------------------------------------------
// Grouped bf16 NT GEMM: C[m][n] = sum over 128-wide K chunks c of
// s(c) * sum_{kk in c} A[m][kk] * B[n][kk], fp32.  Block tile BM (m) x 128
// (n) with four waves of 64 x (BM/2): BM = 128 (2 x 2 waves) for the dgrads
// of large batches (each expert's weights are read once per 128 rows, where
// 64-row tiles made these GEMMs HBM-bound on weight re-reads), BM = 64 (1 x 4
// waves) for small batches and the weight gradients.  Operands staged K-contiguous in LDS (272-byte rows); the
// next 128-wide chunk is loaded into registers while this one computes.
//   DGRAD2: m = rows of an m-tile of one expert (tile list), A = dY (sorted
//     rows, K = H), B = Wd^T of the expert ([I][H]), s = down block scale;
//     epilogue: the activation derivative at the forward's G, U -> dG, dU
//     (bf16, [rows][2I] or [rows][I] gate-less).
//   DGRAD1: A = [dG dU] (K = 2I, or I), B = [Wg Wu]^T ([H][2I]), s = gate or
//     up block scale; epilogue: dx per sorted row (fp32).
//   WGRAD: blockIdx.z = expert; m over the weight rows, n over its inputs,
//     K = the expert's padded row segment of the transposed buffers, s = 1;
//     epilogue: dW[e] (fp32, master layout).
// ---------------------------------------------------------------------------
enum { DGRAD2 = BG_DGRAD2, DGRAD1 = BG_DGRAD1, WGRAD = BG_WGRAD };

// KS: K per LDS stage (128; 64 for the weight gradients, whose K loops are
// short: half the LDS and prefetch registers, more blocks per CU to hide each
// tile's load latency).  Rows are padded by 8 elements against bank conflicts.
template <int BM, int KS>
struct BgTile {
    static constexpr int WR = BM / 64;             // wave rows
    static constexpr int WC = 4 / WR;              // wave columns
    static constexpr int NJ = 128 / WC / 16;       // 16-column n-tiles per wave
    static constexpr int PITCH = KS + 8;           // bf16 elements per LDS row
    static constexpr int SEGS = KS / 8;            // 16-byte segments per row and stage
    static constexpr int QA = BM * SEGS / 256;     // A pieces per thread per stage
    static constexpr int QB = 128 * SEGS / 256;    // B pieces per thread per stage
    static constexpr int OPS_BYTES = (BM + 128) * PITCH * 2;
    // the fp32 tile is staged for its stores in passes of PR rows
    static constexpr int PR = OPS_BYTES >= BM * 132 * 4 ? BM : 32;
    static constexpr int LDS = OPS_BYTES > PR * 132 * 4 ? OPS_BYTES : PR * 132 * 4;
    static_assert(BM % PR == 0 && PR % 16 == 0, "passes cover whole 16-row tiles");
};
template <int MODE, int BM, int KS>
__global__ __launch_bounds__(256) void k_bgemm(BgemmArgs a, int NB)
{
    using TL = BgTile<BM, KS>;
    constexpr int NJ = TL::NJ, PITCH = TL::PITCH, SEGS = TL::SEGS;
    static_assert(MODE == WGRAD || KS == 128, "the dgrads promote once per 128-wide stage");
    extern __shared__ __align__(16) uint16_t smem_bg[];
    uint16_t* As = smem_bg;
    uint16_t* Bs = smem_bg + BM * PITCH;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int wr = w / TL::WC, wc = w % TL::WC;
    int e, row0, rows, kbeg, kend;
    const int nb = blockIdx.x % NB;
    const int n0 = nb * 128;
    int m0 = 0;
    if (MODE == WGRAD) {
        e = blockIdx.z;
        m0 = (blockIdx.x / NB) * BM;
        row0 = 0;
        rows = BM;
        kbeg = a.padoff[e];
        kend = kbeg + ((a.offsets[e + 1] - a.offsets[e] + 31) & ~31);
    } else {
        const int mt = blockIdx.x / NB;
        if (mt >= a.ctrl[0]) return;
        e = a.mt_expert[mt];
        row0 = a.mt_row0[mt];
        rows = min(BM, a.offsets[e + 1] - row0);
        kbeg = 0;
        kend = a.K;
    }
    const uint16_t* Bb = a.B + (size_t)e * a.b_expert;       // WGRAD: bf16 activations
    const uint8_t* Bq = a.Bq + (size_t)e * a.b_expert;       // DGRAD: E4M3 transposed weights
    v4f acc[4][NJ], part[4][NJ];
#pragma unroll
    for (int i = 0; i < 4; i++)
#pragma unroll
        for (int j = 0; j < NJ; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

    // Each thread moves QA A and QB B 16-byte pieces per stage: piece q is
    // row (tid / SEGS) + (256 / SEGS) q, columns 8 * (tid % SEGS)...; the next
    // stage's pieces are loaded into registers while this one computes.  Rows
    // past the end of a DGRAD m-tile and columns past the stage's end are not
    // loaded but read as zero (those rows' products are never stored).
    constexpr int RSTEP = 256 / SEGS;
    uint4 ra[TL::QA], rb[TL::QB];
    uint2 rq[TL::QB];   // DGRAD: the weight pieces as E4M3 bytes, converted when staged
    auto load = [&](int k0) {
        const int kn = min(KS, kend - k0);
        const int sg = tid % SEGS;
        const bool in = sg * 8 < kn;
#pragma unroll
        for (int q = 0; q < TL::QA; q++) {
            const int r = tid / SEGS + RSTEP * q;
            const int ar = MODE == WGRAD ? m0 + r : row0 + min(r, rows - 1);
            ra[q] = in && (MODE == WGRAD || r < rows)
                        ? *reinterpret_cast<const uint4*>(a.A + (size_t)ar * a.lda + k0 + sg * 8)
                        : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int q = 0; q < TL::QB; q++) {
            const int r = tid / SEGS + RSTEP * q;
            if (MODE == WGRAD)
                rb[q] = in ? *reinterpret_cast<const uint4*>(Bb + (size_t)(n0 + r) * a.ldb + k0 + sg * 8)
                           : make_uint4(0, 0, 0, 0);
            else
                rq[q] = in ? *reinterpret_cast<const uint2*>(Bq + (size_t)(n0 + r) * a.ldb + k0 + sg * 8)
                           : make_uint2(0, 0);
        }
    };
    if (kbeg < kend) load(kbeg);
    for (int k0 = kbeg; k0 < kend; k0 += KS) {
        const int kn = min(KS, kend - k0);           // multiple of 32
        __syncthreads();                             // the previous stage's LDS reads are done
        {
            const int sg = tid % SEGS;
#pragma unroll
            for (int q = 0; q < TL::QA; q++)
                *reinterpret_cast<uint4*>(&As[(tid / SEGS + RSTEP * q) * PITCH + sg * 8]) = ra[q];
#pragma unroll
            for (int q = 0; q < TL::QB; q++)
                *reinterpret_cast<uint4*>(&Bs[(tid / SEGS + RSTEP * q) * PITCH + sg * 8]) =
                    MODE == WGRAD ? rb[q] : e4m3x8_to_bf16x8(rq[q]);
        }
        __syncthreads();
        if (k0 + KS < kend) load(k0 + KS);
        if (MODE != WGRAD) {
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++) part[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        }
        for (int ks = 0; ks < kn; ks += 32) {
            bf8 bfr[NJ];
#pragma unroll
            for (int j = 0; j < NJ; j++)
                bfr[j] = *reinterpret_cast<const bf8*>(
                    &Bs[(wc * NJ * 16 + j * 16 + (lane & 15)) * PITCH + ks + 8 * (lane >> 4)]);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const bf8 afr = *reinterpret_cast<const bf8*>(
                    &As[(wr * 64 + i * 16 + (lane & 15)) * PITCH + ks + 8 * (lane >> 4)]);
#pragma unroll
                for (int j = 0; j < NJ; j++) {
                    if (MODE == WGRAD) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], acc[i][j], 0, 0, 0);
                    else part[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[j], part[i][j], 0, 0, 0);
                }
            }
        }
        if (MODE != WGRAD) {
            float s = 1.0f;
            if (MODE == DGRAD2) s = a.blk0[((size_t)e * (a.H / 128) + k0 / 128) * (a.I / 128) + n0 / 128];
            if (MODE == DGRAD1) {
                const int c = k0 / 128, ci = a.I / 128;
                s = c < ci ? a.blk0[((size_t)e * ci + c) * (a.H / 128) + n0 / 128]
                           : a.blk1[((size_t)e * ci + (c - ci)) * (a.H / 128) + n0 / 128];
            }
#pragma unroll
            for (int i = 0; i < 4; i++)
#pragma unroll
                for (int j = 0; j < NJ; j++)
#pragma unroll
                    for (int q = 0; q < 4; q++) acc[i][j][q] = __builtin_fmaf(s, part[i][j][q], acc[i][j][q]);
        }
    }
    // stage the BM x 128 fp32 tile through LDS (the operand buffers reused),
    // PR rows at a time, then store rows with 16-byte writes
    constexpr int PR = TL::PR;
    float* cs = reinterpret_cast<float*>(smem_bg);            // [PR][132]
    for (int pass = 0; pass < BM / PR; pass++) {
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int rl = wr * 64 + i * 16;
            if (rl / PR != pass) continue;
#pragma unroll
            for (int j = 0; j < NJ; j++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    cs[(rl - pass * PR + 4 * (lane >> 4) + q) * 132 + wc * NJ * 16 + j * 16 + (lane & 15)] = acc[i][j][q];
        }
        __syncthreads();
        for (int idx = tid; idx < PR * 32; idx += 256) {
            const int r = pass * PR + (idx >> 5), c4 = (idx & 31) * 4;
            const float4 v = *reinterpret_cast<const float4*>(&cs[(idx >> 5) * 132 + c4]);
            if (MODE == WGRAD) {
                *reinterpret_cast<float4*>(a.dW + ((size_t)e * a.M + m0 + r) * a.N + n0 + c4) = v;
            } else if (r < rows) {
                const size_t row = (size_t)row0 + r;
                if (MODE == DGRAD1) {
                    *reinterpret_cast<float4*>(a.dxs + row * a.H + n0 + c4) = v;
                } else {
                    const float dh[4] = {v.x, v.y, v.z, v.w};
                    const float4 U = *reinterpret_cast<const float4*>(a.u + row * a.I + n0 + c4);
                    const float uu[4] = {U.x, U.y, U.z, U.w};
                    float dg[4], du[4];
                    if (a.act == 0) {
                        const float4 G = *reinterpret_cast<const float4*>(a.g + row * a.I + n0 + c4);
                        const float gg[4] = {G.x, G.y, G.z, G.w};
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            const float sg = 1.0f / (1.0f + expf(-gg[q]));
                            dg[q] = dh[q] * uu[q] * sg * (1.0f + gg[q] * (1.0f - sg));
                            du[q] = dh[q] * gg[q] * sg;
                        }
                    } else {
#pragma unroll
                        for (int q = 0; q < 4; q++) {
                            dg[q] = 0.0f;
                            du[q] = uu[q] > 0.0f ? (a.act == 1 ? 2.0f * uu[q] * dh[q] : dh[q]) : 0.0f;
                        }
                    }
                    const int ld = a.act == 0 ? 2 * a.I : a.I;
                    uint16_t* d = a.dgu + row * ld + n0 + c4;
                    if (a.act == 0) {
                        *reinterpret_cast<uint2*>(d) = make_uint2(bf16x2(dg[0], dg[1]), bf16x2(dg[2], dg[3]));
                        d += a.I;
                    }
                    *reinterpret_cast<uint2*>(d) = make_uint2(bf16x2(du[0], du[1]), bf16x2(du[2], du[3]));
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Weight gradients for large batches, B held in registers: dW_e[m][n] = sum
// over the expert's padded columns c of A[m][c] B[n][c] (both [channel][column]
// bf16, fp32 accumulation, the master layout out).  An expert's padded column
// count Kp (its rows rounded up to 32, ~2.9 x 10^2 at prefill) is short, so a
// tile that loads both operands for every 64 x 128 output moves 3.4 bytes
// through the texture path per byte of fp32 it writes.  Here a block owns 128
// columns n0.. of one expert's dW: each of its four waves keeps the MFMA
// operands of its 32 columns for all of Kp (up to KMAX) in registers, loaded
// once, and the block walks down dW in 128-row tiles, A's rows staged in LDS
// with the next tile's loaded into registers while the current one computes:
// 1.1 bytes read per byte written, with 76 KB of LDS so that two blocks share
// a CU and one's loads and stores overlap the other's products.  Experts with
// more columns take them in KMAX chunks, the B operand reloaded per chunk.
// ---------------------------------------------------------------------------
typedef uint32_t v4u __attribute__((ext_vector_type(4)));   // (a uint4 copy would keep arrays in scratch)
template <int KMAX>
struct WgTile {
    static constexpr int PITCH = KMAX + 8;                  // bf16 per LDS row of A
    static constexpr int NS = KMAX / 32;                    // K steps of 32
    static constexpr int QA = 128 * (KMAX / 8) / 256;       // 16-byte A pieces per thread per tile
    static constexpr int LDS = 128 * PITCH * 2;             // the A tile, reused for the fp32 staging
    static_assert(128 * 132 * 4 <= LDS, "the fp32 tile is staged in the A buffer");
    static_assert((128 * (KMAX / 8)) % 256 == 0 && KMAX % 32 == 0, "tile shape");
};
// Piece q of a 128-row tile of KMAX columns (KMAX/8 16-byte segments per
// row): i = tid + 256 q, row i / (KMAX/8), segment i % (KMAX/8), the quotient
// by a 24-bit multiply and shift (exact for every i of the tile, which the
// static assertion checks; row * ld fits 32 bits as ld < 2^25).  Segments
// at or past klen are clamped to the last one inside it: the copy then moves
// the same 16 bytes to the same place twice.  Indices are recomputed at each
// use (cheap full-rate integer ops) rather than held in registers.
template <int KMAX>
__device__ __forceinline__ void wg_piece(int tid, int q, int klen, uint32_t& row, uint32_t& seg)
{
    constexpr uint32_t SPR = KMAX / 8, MUL = ((1u << 20) + SPR - 1) / SPR;
    static_assert((uint64_t)128 * SPR * (MUL * SPR - (1u << 20)) < (1u << 20), "exact quotient for i < 128 SPR");
    const uint32_t i = (uint32_t)tid + 256u * q;
    row = __umul24(i, MUL) >> 20;
    seg = min(i - row * SPR, (uint32_t)klen / 8u - 1u);
}
template <int KMAX, int Q>
__device__ __forceinline__ void wg_fetch(v4u (&r)[Q], const uint16_t* base, int ld, int row0, int c0, int klen, int tid)
{
    asm volatile("" : "+v"(tid));                          // piece indices recomputed here, not held
    const uint16_t* b = base + (size_t)row0 * ld + c0;     // uniform
#pragma unroll
    for (int q = 0; q < Q; q++) {
        uint32_t row, seg;
        wg_piece<KMAX>(tid, q, klen, row, seg);
        r[q] = *reinterpret_cast<const v4u*>(b + (row * (uint32_t)ld + seg * 8u));
    }
}
template <int KMAX, int PITCH, int Q>
__device__ __forceinline__ void wg_put(uint16_t* dst, const v4u (&r)[Q], int klen, int tid)
{
    asm volatile("" : "+v"(tid));
#pragma unroll
    for (int q = 0; q < Q; q++) {
        uint32_t row, seg;
        wg_piece<KMAX>(tid, q, klen, row, seg);
        *reinterpret_cast<v4u*>(&dst[row * PITCH + seg * 8u]) = r[q];
    }
}
template <int KMAX>
__global__ __launch_bounds__(256) void k_wgrad(BgemmArgs a)
{
    using TL = WgTile<KMAX>;
    constexpr int PITCH = TL::PITCH, NS = TL::NS;
    extern __shared__ __align__(16) uint16_t smem_wg[];
    uint16_t* As = smem_wg;
    float* cs = reinterpret_cast<float*>(smem_wg);           // [128][132] fp32 staging
    const int e = blockIdx.y, n0 = blockIdx.x * 128;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int cbeg = a.padoff[e];
    const int Kp = (a.offsets[e + 1] - a.offsets[e] + 31) & ~31;
    const int nkc = Kp > 0 ? (Kp + KMAX - 1) / KMAX : 1;      // an expert without rows runs one empty chunk: zeros
    const int items = (a.M / 128) * nkc;                      // (128-row tile, K chunk), chunk fastest
    const uint16_t* Bb = a.B + (size_t)e * a.b_expert;
    // this wave's B operand: columns n0 + 32w + 16j + (lane % 16), 8 K values
    // from 32s + 8 (lane / 16) of the chunk
    const uint16_t* brow[2] = {Bb + (size_t)(n0 + 32 * w + (lane & 15)) * a.ldb + 8 * (lane >> 4),
                               Bb + (size_t)(n0 + 32 * w + 16 + (lane & 15)) * a.ldb + 8 * (lane >> 4)};
    bf8 bfr[NS][2];
    auto load_b = [&](int c0, int klen) {
#pragma unroll
        for (int st = 0; st < NS; st++)
#pragma unroll
            for (int j = 0; j < 2; j++)
                if (32 * st < klen) bfr[st][j] = *reinterpret_cast<const bf8*>(brow[j] + c0 + 32 * st);
        // waited for here: a B reload is conditional, and a wait left to the
        // compiler at the first product would also wait for the A prefetch
        __builtin_amdgcn_s_waitcnt(0xF70);   // vmcnt(0)
    };
    v4u ra[TL::QA];
    if (Kp > 0) {
        load_b(cbeg, min(KMAX, Kp));
        wg_fetch<KMAX>(ra, a.A, a.lda, 0, cbeg, min(KMAX, Kp), tid);
    }
    v4f acc[8][2];
    for (int it = 0; it < items; it++) {
        const int mt = it / nkc, kc = it % nkc;
        const int klen = Kp > 0 ? min(KMAX, Kp - kc * KMAX) : 0;
        if (kc == 0)
#pragma unroll
            for (int i = 0; i < 8; i++)
#pragma unroll
                for (int j = 0; j < 2; j++) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};
        __syncthreads();                                      // As free: the last item's reads and stores are done
        if (klen > 0) {
            wg_put<KMAX, PITCH>(As, ra, klen, tid);
            if (nkc > 1 && kc > 0) load_b(cbeg + kc * KMAX, klen);
        }
        __syncthreads();
        if (it + 1 < items && Kp > 0) {
            const int mt1 = (it + 1) / nkc, kc1 = (it + 1) % nkc;
            wg_fetch<KMAX>(ra, a.A, a.lda, mt1 * 128, cbeg + kc1 * KMAX, min(KMAX, Kp - kc1 * KMAX), tid);
        }
#pragma unroll
        for (int st = 0; st < NS; st++) {
            if (32 * st >= klen) break;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const bf8 afr = *reinterpret_cast<const bf8*>(&As[(i * 16 + (lane & 15)) * PITCH + 32 * st + 8 * (lane >> 4)]);
#pragma unroll
                for (int j = 0; j < 2; j++)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[st][j], acc[i][j], 0, 0, 0);
            }
        }
        if (kc + 1 < nkc) continue;                         // the next chunk's B is loaded at its start
        // the 128 x 128 fp32 tile through LDS, then 16-byte row stores
        __syncthreads();
#pragma unroll
        for (int i = 0; i < 8; i++)
#pragma unroll
            for (int j = 0; j < 2; j++)
#pragma unroll
                for (int q = 0; q < 4; q++)
                    cs[(i * 16 + 4 * (lane >> 4) + q) * 132 + 32 * w + j * 16 + (lane & 15)] = acc[i][j][q];
        __syncthreads();
#pragma unroll 1
        for (int q0 = 0; q0 < 16; q0 += 4) {
            float4 v[4];
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int r = (tid >> 5) + 8 * (q0 + q);
                v[q] = *reinterpret_cast<const float4*>(&cs[r * 132 + (tid & 31) * 4]);
            }
#pragma unroll
            for (int q = 0; q < 4; q++) {
                const int r = (tid >> 5) + 8 * (q0 + q);
                *reinterpret_cast<float4*>(a.dW + ((size_t)e * a.M + mt * 128 + r) * a.N + n0 + (tid & 31) * 4) = v[q];
            }
        }
        // a chunked expert's next tile starts again at chunk 0: its B operand
        if (nkc > 1 && it + 1 < items) load_b(cbeg, min(KMAX, Kp));
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
hipError_t launch_bwd_combine(int T, int H, int k, const uint16_t* dout, const float* w, const uint16_t* y,
                              const int32_t* pair_pos, uint16_t* dys, float* dw, hipStream_t s)
{
    if (T == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bwd_combine, dim3((unsigned)(T * k)), dim3(256), 0, s, H, k, dout, w, y, pair_pos, dys, dw);
    return hipGetLastError();
}

hipError_t launch_weights_t(int E, int N, int K, const uint8_t* fp4, const uint8_t* e8, uint8_t* out, int ldo,
                            int nofs, size_t out_expert_stride, hipStream_t s)
{
    const size_t blocks = (size_t)E * (N / 64) * (K / 128);
    hipLaunchKernelGGL(k_weights_t, dim3((unsigned)blocks), dim3(256), 0, s, N, K, fp4, e8, out, ldo, nofs,
                       out_expert_stride);
    return hipGetLastError();
}

hipError_t launch_pad_offsets(int E, const int32_t* off, int32_t* padoff, hipStream_t s)
{
    hipLaunchKernelGGL(k_pad_offsets, dim3(1), dim3(1024), 0, s, E, off, padoff);
    return hipGetLastError();
}

hipError_t launch_bwd_transpose(int mode, int C, int E, int k, int max_cols, const int32_t* off,
                                const int32_t* padoff, const int32_t* sorted_pair, const uint16_t* src16,
                                const uint8_t* q8, const float* qs, int qs_stride, uint16_t* dst, int ldd,
                                hipStream_t s)
{
    const dim3 grid((unsigned)((max_cols + 63) / 64), (unsigned)(C / 64));
    if (mode == 0)
        hipLaunchKernelGGL(k_bwd_transpose<0>, grid, dim3(256), 0, s, C, E, k, off, padoff, sorted_pair, src16, q8,
                           qs, qs_stride, dst, ldd);
    else if (mode == 1)
        hipLaunchKernelGGL(k_bwd_transpose<1>, grid, dim3(256), 0, s, C, E, k, off, padoff, sorted_pair, src16, q8,
                           qs, qs_stride, dst, ldd);
    else
        hipLaunchKernelGGL(k_bwd_transpose<2>, grid, dim3(256), 0, s, C, E, k, off, padoff, sorted_pair, src16, q8,
                           qs, qs_stride, dst, ldd);
    return hipGetLastError();
}

hipError_t launch_bwd_unpermute(int T, int H, int k, const int32_t* pair_pos, const float* dxs, float* dx,
                                hipStream_t s)
{
    const size_t n = (size_t)T * H / 4;
    if (n == 0) return hipSuccess;
    hipLaunchKernelGGL(k_bwd_unpermute, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, T, H, k, pair_pos, dxs, dx);
    return hipGetLastError();
}

template <int MODE, int BM, int KS = 128>
static hipError_t launch_bgemm_t(const BgemmArgs& a, dim3 grid, int NB, hipStream_t s)
{
    constexpr int LDS = BgTile<BM, KS>::LDS;
    static bool lds_ok = false;
    if (!lds_ok) {
        if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_bgemm<MODE, BM, KS>),
                                hipFuncAttributeMaxDynamicSharedMemorySize, LDS) != hipSuccess)
            return hipErrorInvalidValue;
        lds_ok = true;
    }
    hipLaunchKernelGGL((k_bgemm<MODE, BM, KS>), grid, dim3(256), LDS, s, a, NB);
    return hipGetLastError();
}

// DGRAD modes: bm (64 or 128) is the row count of the m-tiles in the list;
// WGRAD: bm = 128 selects k_wgrad.
hipError_t launch_bgemm(int mode, int bm, const BgemmArgs& a, int n_mt_bound, int E, hipStream_t s)
{
    const int NB = a.N / 128;
    if (mode == WGRAD) {
        if (E == 0) return hipSuccess;
        if (bm != 128) return launch_bgemm_t<WGRAD, 64, 64>(a, dim3((unsigned)((a.M / 64) * NB), 1, (unsigned)E), NB, s);
        constexpr int KMAX = 288;
        constexpr int LDS = WgTile<KMAX>::LDS;
        static bool lds_ok = false;
        if (!lds_ok) {
            if (hipFuncSetAttribute(reinterpret_cast<const void*>(k_wgrad<KMAX>),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, LDS) != hipSuccess)
                return hipErrorInvalidValue;
            lds_ok = true;
        }
        hipLaunchKernelGGL(k_wgrad<KMAX>, dim3((unsigned)NB, (unsigned)E), dim3(256), LDS, s, a);
        return hipGetLastError();
    }
    const dim3 grid((unsigned)(n_mt_bound * NB));
    if (bm == 128)
        return mode == DGRAD2 ? launch_bgemm_t<DGRAD2, 128>(a, grid, NB, s) : launch_bgemm_t<DGRAD1, 128>(a, grid, NB, s);
    return mode == DGRAD2 ? launch_bgemm_t<DGRAD2, 64>(a, grid, NB, s) : launch_bgemm_t<DGRAD1, 64>(a, grid, NB, s);
}

}  // namespace v4moe
