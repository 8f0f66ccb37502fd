// v4moe_kernels.hip -- HIP kernels of the MoE layer forward for gfx950.
//
// Sources (cited by short tag and section):
//   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
//   P2 = "DeepSeek V4架构学习笔记"
//
// Kernels, in the order a layer forward runs them:
//   k_route_logits / k_route_logits_any + k_route_select, or k_route_hash
//                                    routing (P2, DeepSeekMoE notes)
//   k_quant_x                        FP8 dispatch payload (P1 §1.4)
//   k_perm_small, or k_perm_pass<count> + k_perm_scan + k_perm_pass<positions>
//                                    expert histogram, offsets, stable positions
//   k_build_tiles                    m-tile list and the wave-ordered work queue
//   k_ffn<1,...>, k_ffn<2,...>       linear1+SwiGLU+requant, linear2+scatter
//   k_ffn_persistent<...>            the same tiles, wave-scheduled in one launch
//                                    (m-tiles of up to 64 rows)
//   k_combine                        fixed-order weighted un-permute
// plus the offline k_prepack and the test export k_dequant_export.
//
// Every tile of linear1/linear2 runs the same per-element arithmetic whatever
// the tile shape or the schedule: one 16x16x128 block-scaled FP8 x FP4 MFMA
// per 128-wide K chunk, then acc = fma(xs*blk, P, acc) with chunks in
// increasing order.  A row's result therefore does not depend on which rows
// share its tile (P1 §3.1, batch invariance; no split-K) and never on timing
// (P1 §3.2: no atomic accumulation anywhere).
#include "v4moe_device.h"
#include "v4moe_internal.h"

#include <limits.h>
#include <type_traits>

namespace v4moe {

// ---------------------------------------------------------------------------
// Routing
// ---------------------------------------------------------------------------

// Wait until at most N of this wave's vector memory operations are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt is 6 bits");
    __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Direct-to-LDS copy: each lane moves 16 bytes from its own global address to
// lds_base + lane*16 (lds_base wave-uniform, in M0); lanes outside EXEC do not
// write.  As inline asm it is invisible to the compiler's wait insertion:
// completion is awaited with an explicit wait_vm.
__device__ __forceinline__ void dma16(const void* g, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                 :: "v"(g), "s"(lds_base) : "memory", "m0");
}

// A value known to be equal in every lane, moved to scalar registers.
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
template <typename T>
__device__ __forceinline__ T* uniform(T* p)
{
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<T*>((uintptr_t)(((uint64_t)hi << 32) | lo));
}
// One 128-channel group of the FP8 dispatch payload held by 16 consecutive
// lanes, 8 channels each (f): amax over the group, s = amax / 448 (1 for an
// all-zero group), codes = E4M3(f / s).  Every lane of the 16 must call it;
// lanes with store = false only take part in the reduction.  The scale goes
// to *scale when that pointer is not null.
__device__ __forceinline__ void x_quant_group(const float (&f)[8], bool store, uint8_t* q8, float* scale)
{
    float amax = 0.0f;
#pragma unroll
    for (int u = 0; u < 8; u++) amax = fmaxf(amax, fabsf(f[u]));
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
    if (!store) return;
    const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
    const uint32_t lo = e4m3x2(f[0] / s, f[1] / s) | (e4m3x2(f[2] / s, f[3] / s) << 16);
    const uint32_t hi = e4m3x2(f[4] / s, f[5] / s) | (e4m3x2(f[6] / s, f[7] / s) << 16);
    *reinterpret_cast<uint2*>(q8) = make_uint2(lo, hi);
    if (scale) *scale = s;
}

// Router logits, every variant: z[t][e] is one fp32 fma chain over h
// ascending from +0 (x exact as float), plus the optional bias as one fp32 add
// afterwards.  The variants differ only in which chains a lane runs and how the
// operands reach it.
//
// k_route_logits: lane = TS tokens x ES experts of independent chains (tokens
// t0 + l + 64*i, i < TS; the ES experts of its wave).  Block = 4 waves, 64*TS
// tokens x 4*ES experts.  The block's slice of W_r is staged through LDS HC
// rows at a time, transposed to expert-major rows (padded by 4 floats against
// bank conflicts), so one broadcast LDS read gives four consecutive h of one
// expert; the next slice is loaded into registers while the current one is
// used.  With XL the tokens' x rows are staged too, by direct-to-LDS loads
// issued a stage ahead (rows padded by 16 bytes); otherwise each lane reads its
// x rows from global memory one step ahead.  z is [T][E].  Needs E % (4*ES) ==
// 0 and H % HC == 0.
template <int TS, int ES, int HC, bool XL>
__global__ __launch_bounds__(256) void k_route_logits(int T, int H, int E,
                                                      const uint16_t* __restrict__ x,
                                                      const float* __restrict__ wr,
                                                      const float* __restrict__ bias,
                                                      float* __restrict__ z)
{
    constexpr int EB = 4 * ES;               // experts per block
    constexpr int PITCH = HC + 4;            // floats per expert row in LDS
    constexpr int NV = HC * EB / 4;          // float4 of W per stage
    constexpr int LD = (NV + 255) / 256;     // float4 loads per thread per stage
    constexpr int XP = HC / 8 + 1;           // uint4 per staged x row
    constexpr int NSLOT = XL ? 64 * TS * XP : 0;      // uint4 slots of staged x per stage
    constexpr int HS = XL && TS * ES < 8 ? 64 : 8;  // h per inner step (one LDS wait per step; eight chains'
                                                    // W and x reads of 64 h would not fit the registers)
    __shared__ __align__(16) float wt[2][EB * PITCH];
    __shared__ __align__(16) uint4 xt[XL ? 2 : 1][XL ? 64 * TS * XP : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int t0 = blockIdx.x * 64 * TS;
    const int eb0 = blockIdx.y * EB;
    const int nst = H / HC;

    // staging: float4 f of the [HC][EB] slice = row f / (EB/4), experts 4*(f % (EB/4)) .. +3;
    // uint4 g of the x slice = token row g / (HC/8), 8 h at column g % (HC/8)
    float4 nxt[LD];
    // x slice of stage st into buffer buf: DMA k (of this wave: k = w, w+4, ...)
    // fills slots 64k .. 64k+63; slot = row*XP + col, the padding column
    // repeats the last real one.
    auto dma_x = [&](int st, int buf) {
        if (XL) {
            const uint32_t base = (uint32_t)(uintptr_t)&xt[XL ? buf : 0][0];
            for (int k = w; k * 64 < NSLOT; k += 4) {
                const int slot = 64 * k + lane;
                const int row = slot / XP, col = min(slot % XP, HC / 8 - 1);
                if (slot < NSLOT)
                    dma16(x + (size_t)min(t0 + row, T - 1) * H + st * HC + col * 8,
                          __builtin_amdgcn_readfirstlane(base + k * 1024));
            }
        }
    };
    auto load_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < LD; i++) {
            const int f = tid + 256 * i;
            if (f < NV)
                nxt[i] = *reinterpret_cast<const float4*>(wr + (size_t)(st * HC + f / (EB / 4)) * E + eb0 +
                                                          4 * (f % (EB / 4)));
        }
    };
    auto store_stage = [&](int buf) {
#pragma unroll
        for (int i = 0; i < LD; i++) {
            const int f = tid + 256 * i;
            if (f < NV) {
                const int h = f / (EB / 4), e4 = 4 * (f % (EB / 4));
                wt[buf][(e4 + 0) * PITCH + h] = nxt[i].x;
                wt[buf][(e4 + 1) * PITCH + h] = nxt[i].y;
                wt[buf][(e4 + 2) * PITCH + h] = nxt[i].z;
                wt[buf][(e4 + 3) * PITCH + h] = nxt[i].w;
            }
        }
    };
    dma_x(0, 0);
    load_stage(0);
    store_stage(0);
    wait_vm<0>();
    __syncthreads();

    const uint4* xp[TS];
#pragma unroll
    for (int i = 0; i < TS; i++) xp[i] = reinterpret_cast<const uint4*>(x + (size_t)min(t0 + lane + 64 * i, T - 1) * H);
    float acc[TS][ES];
#pragma unroll
    for (int i = 0; i < TS; i++)
#pragma unroll
        for (int j = 0; j < ES; j++) acc[i][j] = 0.0f;

    // x of 8 consecutive h of token i, for the step starting at stage-relative h
    auto xload = [&](int s, int i, int h) -> uint4 {
        if (XL) return xt[XL ? (s & 1) : 0][(lane + 64 * i) * XP + h / 8];
        const int g = s * HC + h;
        return xp[i][(g < H ? g : H - 8) / 8];
    };
    for (int s = 0; s < nst; s++) {
        if (s + 1 < nst) {
            dma_x(s + 1, (s + 1) & 1);
            load_stage(s + 1);
        }
        const float* wb = wt[s & 1] + w * ES * PITCH;
        float4 wc[ES][HS / 4];
        uint4 xc[TS][HS / 8];
#pragma unroll
        for (int j = 0; j < ES; j++)
#pragma unroll
            for (int v = 0; v < HS / 4; v++) wc[j][v] = *reinterpret_cast<const float4*>(wb + j * PITCH + 4 * v);
#pragma unroll
        for (int i = 0; i < TS; i++)
#pragma unroll
            for (int v = 0; v < HS / 8; v++) xc[i][v] = xload(s, i, 8 * v);
#pragma unroll 1
        for (int h = 0; h < HC; h += HS) {
            // operands of the next step (this stage's last step re-reads its own)
            const int hn = h + HS < HC ? h + HS : h;
            float4 wn[ES][HS / 4];
            uint4 xn[TS][HS / 8];
#pragma unroll
            for (int j = 0; j < ES; j++)
#pragma unroll
                for (int v = 0; v < HS / 4; v++) wn[j][v] = *reinterpret_cast<const float4*>(wb + j * PITCH + hn + 4 * v);
#pragma unroll
            for (int i = 0; i < TS; i++)
#pragma unroll
                for (int v = 0; v < HS / 8; v++) xn[i][v] = xload(s, i, (XL ? hn : h + HS) + 8 * v);
#pragma unroll
            for (int u = 0; u < HS; u++) {
#pragma unroll
                for (int i = 0; i < TS; i++) {
                    const uint4 xq = xc[i][u / 8];
                    const int k8 = u & 7;
                    const uint32_t q = k8 < 2 ? xq.x : k8 < 4 ? xq.y : k8 < 6 ? xq.z : xq.w;
                    const float xv = __uint_as_float((u & 1) ? (q & 0xFFFF0000u) : (q << 16));
#pragma unroll
                    for (int j = 0; j < ES; j++) {
                        const float4 v = wc[j][u >> 2];
                        const float wv = (u & 3) == 0 ? v.x : (u & 3) == 1 ? v.y : (u & 3) == 2 ? v.z : v.w;
                        acc[i][j] = __builtin_fmaf(xv, wv, acc[i][j]);
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < ES; j++)
#pragma unroll
                for (int v = 0; v < HS / 4; v++) wc[j][v] = wn[j][v];
#pragma unroll
            for (int i = 0; i < TS; i++)
#pragma unroll
                for (int v = 0; v < HS / 8; v++) xc[i][v] = xn[i][v];
        }
        if (s + 1 < nst) store_stage((s + 1) & 1);
        if (XL) wait_vm<0>();
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TS; i++) {
        const int t = t0 + lane + 64 * i;
        if (t < T) {
#pragma unroll
            for (int j = 0; j < ES; j++) {
                const int e = eb0 + w * ES + j;
                float v = acc[i][j];
                if (bias) v = v + bias[e];
                z[(size_t)t * E + e] = v;
            }
        }
    }
}

// k_route_lane: for batches too small to fill the chip with several chains
// per lane, where a 4096-long chain is latency-bound (a dependent fp32 fma
// takes about 1.5 issue slots) and the time goes to getting operands to it.
// Lane = one chain: wave = EL experts x 64/EL tokens; block = NTW such waves
// plus one producer wave.  The producer issues every global load of the block
// as a direct-to-LDS load NS-1 stages of RH rows ahead (the W_r slice, rows
// of EL experts, natural [h][e] layout; the block's x rows as bf16), waits for
// a stage's loads, converts its x to fp32 in LDS and releases the stage with
// one barrier.  The consumer waves do nothing but the chain: per step of 16 h
// they read 16 W values (lanes of one expert share each read) and four fp32
// x values per token (lanes of one token share those), the reads of the next
// step issued before the fmas of the current one.  Small EL keeps the W slice
// a block streams through its CU small.  Needs E % 4 == 0 and H % RH == 0;
// lanes past E read clamped columns and store nothing.
template <int EL, int NTW, int RH, int NS>
__global__ __launch_bounds__(64 * (NTW + 1)) void k_route_lane(int T, int H, int E, const uint16_t* __restrict__ x,
                                                             const float* __restrict__ wr,
                                                             const float* __restrict__ bias, float* __restrict__ z,
                                                             uint8_t* __restrict__ xq, float* __restrict__ xs)
{
    constexpr int TPW = 64 / EL;                 // tokens per consumer wave
    constexpr int NTOK = NTW * TPW;              // tokens per block
    constexpr int SPR = EL / 4;                  // 16-byte segments per W row
    constexpr int RPD = 64 / SPR;                // W rows per 1 KiB load
    constexpr int WD = RH / RPD;                 // W loads per stage
    constexpr int XSEG = RH / 8;                 // 16-byte x segments per token row per stage
    constexpr int XD = (NTOK * XSEG + 63) / 64;  // x loads per stage
    constexpr int OPS = WD + XD;                 // producer loads per stage
    constexpr int HS = 16;                       // h per consumer step
    static_assert(EL % 4 == 0 && 64 % EL == 0 && RH % RPD == 0 && RH % (2 * HS) == 0, "stage shape");
    static_assert(NS >= 2 && NS <= 4 && OPS * (NS - 2) < 64, "loads in flight fit the counter");
    __shared__ __align__(16) float wl[NS][RH * EL];
    __shared__ __align__(16) uint4 xst[NS][XD * 64];
    __shared__ __align__(16) float xf[NS][NTOK][RH];
    const int tid = threadIdx.x, lane = tid & 63;
    const int w = uniform(tid >> 6);
    const int neg = (E + EL - 1) / EL;
    const int eg = blockIdx.x % neg, tg = blockIdx.x / neg;
    const int e0 = eg * EL, t0 = tg * NTOK;
    const int nst = H / RH;

    if (w == NTW) {
        // ---- producer ----
        const int ccol = min(e0 + 4 * (lane % SPR), E - 4);
        auto issue = [&](int st) {
            const int slot = st % NS;
            const uint32_t wbase = (uint32_t)(uintptr_t)&wl[slot][0];
#pragma unroll
            for (int k = 0; k < WD; k++)   // rows k*RPD + lane/SPR
                dma16(wr + (size_t)(st * RH + k * RPD + lane / SPR) * E + ccol, uniform((int)(wbase + k * 1024)));
            const uint32_t xbase = (uint32_t)(uintptr_t)&xst[slot][0];
#pragma unroll
            for (int k = 0; k < XD; k++) { // segment g: token g / XSEG (the last one repeated past the end)
                const int g = min(64 * k + lane, NTOK * XSEG - 1);
                const int t = min(t0 + g / XSEG, T - 1);
                dma16(x + (size_t)t * H + st * RH + (g % XSEG) * 8, uniform((int)(xbase + k * 1024)));
            }
        };
        for (int u = 0; u < NS - 1; u++)
            if (u < nst) issue(u);
        for (int s = 0; s < nst; s++) {
            // stage s has landed; later stages may still be in flight
            constexpr int A2 = NS - 2 >= 2 ? 2 * OPS : 0;
            const int ahead = min(NS - 2, nst - 1 - s);
            if (ahead >= 2) wait_vm<A2>(); else if (ahead == 1) wait_vm<OPS>(); else wait_vm<0>();
            const int slot = s % NS;
            // with xq: the stages s = eg (mod groups of experts) of the block's
            // tokens also get their FP8 dispatch payload here (x_quant_group:
            // 16 lanes per 128-channel group), so each is written exactly once
            const bool quant = xq != nullptr && s % neg == eg;
            for (int g = lane; g < NTOK * XSEG; g += 64) {
                const uint4 q = xst[slot][g];
                float f[8] = {bf16_to_f32(q.x & 0xFFFFu), bf16_to_f32(q.x >> 16), bf16_to_f32(q.y & 0xFFFFu),
                              bf16_to_f32(q.y >> 16), bf16_to_f32(q.z & 0xFFFFu), bf16_to_f32(q.z >> 16),
                              bf16_to_f32(q.w & 0xFFFFu), bf16_to_f32(q.w >> 16)};
                float* d = &xf[slot][g / XSEG][(g % XSEG) * 8];
                *reinterpret_cast<float4*>(d) = make_float4(f[0], f[1], f[2], f[3]);
                *reinterpret_cast<float4*>(d + 4) = make_float4(f[4], f[5], f[6], f[7]);
                if (quant) {
                    const int t = t0 + g / XSEG;
                    const size_t off = (size_t)min(t, T - 1) * H + (size_t)s * RH + (g % XSEG) * 8;
                    x_quant_group(f, t < T, xq + off, t < T && (g & 15) == 0 ? xs + off / 128 : nullptr);
                }
            }
            __syncthreads();
            // slot (s-1) % NS is free: every consumer finished stage s-1 before this barrier
            if (s + NS - 1 < nst) issue(s + NS - 1);
        }
        return;
    }
    // ---- consumers: one barrier per stage, the producer's matching one ----
    const int el = lane % EL, tl = lane / EL;
    float acc = 0.0f;
    for (int s = 0; s < nst; s++) {
        __syncthreads();
        const int slot = s % NS;
        const float* wb = &wl[slot][el];
        const float* xb = &xf[slot][w * TPW + tl][0];
        // two register sets in turn: the reads of the next step are issued
        // before the fmas of the current one, with no register copies
        float wA[HS], wB[HS];
        float4 xA[HS / 4], xB[HS / 4];
        auto ld = [&](float (&wv)[HS], float4 (&xv)[HS / 4], int h) {
#pragma unroll
            for (int u = 0; u < HS; u++) wv[u] = wb[(h + u) * EL];
#pragma unroll
            for (int v = 0; v < HS / 4; v++) xv[v] = *reinterpret_cast<const float4*>(xb + h + 4 * v);
        };
        auto mac = [&](const float (&wv)[HS], const float4 (&xv)[HS / 4]) {
#pragma unroll
            for (int v = 0; v < HS / 4; v++) {
                acc = __builtin_fmaf(xv[v].x, wv[4 * v + 0], acc);
                acc = __builtin_fmaf(xv[v].y, wv[4 * v + 1], acc);
                acc = __builtin_fmaf(xv[v].z, wv[4 * v + 2], acc);
                acc = __builtin_fmaf(xv[v].w, wv[4 * v + 3], acc);
            }
            // the step's chain is complete here: later reads are not hoisted
            // above it, nor its fmas sunk below them
            asm volatile("" : "+v"(acc)::"memory");
        };
        ld(wA, xA, 0);
#pragma unroll
        for (int h = 0; h < RH; h += 2 * HS) {
            ld(wB, xB, h + HS);
            mac(wA, xA);
            if (h + 2 * HS < RH) ld(wA, xA, h + 2 * HS);
            mac(wB, xB);
        }
    }
    const int e = e0 + el, t = t0 + w * TPW + tl;
    if (e < E && t < T) z[(size_t)t * E + e] = bias ? acc + bias[e] : acc;
}

// The same logits for any E: one thread per (token, expert).
__global__ __launch_bounds__(256) void k_route_logits_any(int T, int H, int E, const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          const float* __restrict__ bias, float* __restrict__ z)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= (size_t)T * E) return;
    const int t = (int)(i / E), e = (int)(i % E);
    float acc = 0.0f;
    for (int h = 0; h < H; h++) acc = __builtin_fmaf(bf16_to_f32(x[(size_t)t * H + h]), wr[(size_t)h * E + e], acc);
    if (bias) acc = acc + bias[e];
    z[i] = acc;
}

// Order-preserving map of fp32 bits to uint32 (finite values; -0 below +0,
// which the logits never hold: their sums start from +0) and its inverse.
__device__ __forceinline__ uint32_t float_order_key(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float float_from_order_key(uint32_t u)
{
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}
// One DPP move of a 64-bit value (both halves with the same lane pattern).
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v)
{
    const uint32_t hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)(v >> 32), CTRL, 0xF, 0xF, false);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)(uint32_t)v, CTRL, 0xF, 0xF, false);
    return ((uint64_t)hi << 32) | lo;
}
// Maximum of a 64-bit key over the whole wave (every lane active), returned to
// every lane: within each 16-lane row by DPP (quad xor 1, quad xor 2, half-row
// mirror, row mirror), then across the four rows by reading lanes 0/16/32/48.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t v)
{
    uint64_t o;
    o = dpp_u64<0xB1>(v);  v = o > v ? o : v;    // quad_perm [1,0,3,2]
    o = dpp_u64<0x4E>(v);  v = o > v ? o : v;    // quad_perm [2,3,0,1]
    o = dpp_u64<0x141>(v); v = o > v ? o : v;    // row_half_mirror
    o = dpp_u64<0x140>(v); v = o > v ? o : v;    // row_mirror
    uint64_t r = 0;
#pragma unroll
    for (int row = 0; row < 4; row++) {
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 16 * row);
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 16 * row);
        const uint64_t w = ((uint64_t)hi << 32) | lo;
        r = w > r ? w : r;
    }
    return r;
}

// Top-k per token (one wave per token): the k largest logits, the lower expert
// id winning ties, slot j = j-th pick; then lanes 0..k-1 compute the affinity
// sqrt(softplus(z)) and the weights normalised over the k picks.  z is [T][E];
// lane l holds experts l + 64q, q < NQ (NQ*64 >= E).  Each lane keeps the
// largest key of its experts not yet picked; a round takes the wave maximum
// of those, and only the lane that held the pick finds its next best.
template <int NQ>
__device__ __forceinline__ void select_token(int t, int lane, int E, int k, const float* __restrict__ zg,
                                             int32_t* __restrict__ ids, float* __restrict__ wts)
{
    const float* z = zg + (size_t)t * E;
    // key = order-preserving bits of z above the complemented id: the largest
    // key is the largest z, the lower id on equal z; 0 = none (a real key has
    // ~id != 0 in its low half)
    uint64_t cand[NQ];
#pragma unroll
    for (int q = 0; q < NQ; q++) {
        const int e = lane + 64 * q;
        cand[q] = e < E ? ((uint64_t)float_order_key(z[e]) << 32) | (uint32_t)~e : 0;
    }
    auto best_of = [&]() {
        uint64_t b = 0;
#pragma unroll
        for (int q = 0; q < NQ; q++) b = cand[q] > b ? cand[q] : b;
        return b;
    };
    uint64_t best = best_of();
    float my_z = 0.0f;
    int my_e = 0;
    for (int j = 0; j < k; j++) {
        const uint64_t key = wave_max_key(best);
        const int be = (int)~(uint32_t)key;
        if ((be & 63) == lane) {
#pragma unroll
            for (int q = 0; q < NQ; q++)
                if (q == (be >> 6)) cand[q] = 0;
            best = best_of();
        }
        if (lane == j) { my_z = float_from_order_key((uint32_t)(key >> 32)); my_e = be; }
    }
    // affinity sqrt(softplus(z)), softplus(z) = max(z,0) + log1p(exp(-|z|))
    const float a = sqrtf(fmaxf(my_z, 0.0f) + log1pf(expf(-fabsf(my_z))));
    float sum = 0.0f;
    for (int j = 0; j < k; j++) sum += __shfl(a, j);
    if (lane < k) {
        ids[(size_t)t * k + lane] = my_e;
        wts[(size_t)t * k + lane] = sum > 0.0f ? a / sum : 1.0f / (float)k;
    }
}
template <int NQ>
__global__ __launch_bounds__(256) void k_route_select(int T, int E, int k, const float* __restrict__ zg,
                                                      int32_t* __restrict__ ids, float* __restrict__ wts)
{
    const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= T) return;
    select_token<NQ>(t, threadIdx.x & 63, E, k, zg, ids, wts);
}

// Hash routing: expert_j = splitmix64(id*k + j) mod E, +1 mod E past repeats.
__global__ __launch_bounds__(256) void k_route_hash(int T, int E, int k,
                                                    const int64_t* __restrict__ tids,
                                                    int32_t* __restrict__ ids,
                                                    float* __restrict__ wts)
{
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t >= T) return;
    const uint64_t id = tids ? (uint64_t)tids[t] : (uint64_t)t;
    int32_t* o = ids + (size_t)t * k;
    for (int j = 0; j < k; j++) {
        int c = (int)(splitmix64(id * (uint64_t)k + (uint64_t)j) % (uint64_t)E);
        for (;;) {
            bool dup = false;
            for (int i = 0; i < j; i++) dup |= (o[i] == c);
            if (!dup) break;
            c = (c + 1 == E) ? 0 : c + 1;
        }
        o[j] = c;
        wts[(size_t)t * k + j] = 1.0f / (float)k;
    }
}

// ---------------------------------------------------------------------------
// FP8 dispatch payload: x -> (xq, xs) per token and 128-channel group.
// 16 consecutive threads own one group (8 channels each, one 16-byte load).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_quant_x(int T, int H, const uint16_t* __restrict__ x,
                                                 uint8_t* __restrict__ xq, float* __restrict__ xs)
{
    const size_t total = (size_t)T * H / 8;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    const bool ok = idx < total;
    float f[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    if (ok) {
        uint4 v = *reinterpret_cast<const uint4*>(x + idx * 8);
        uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; u++) {
            f[2 * u] = bf16_to_f32(q[u] & 0xFFFFu);
            f[2 * u + 1] = bf16_to_f32(q[u] >> 16);
        }
    }
    x_quant_group(f, ok, xq + (ok ? idx * 8 : 0), ok && (idx & 15) == 0 ? xs + idx / 16 : nullptr);
}

// ---------------------------------------------------------------------------
// Expert-sorted permutation (stable counting sort of pair ids by expert).
// Each 64-thread block owns kPermChunk consecutive pairs.  Within a wave the
// lanes holding the same expert find each other with one ballot per id bit;
// a lane's rank among them is a popcount of the lower lanes, so positions
// follow pair order exactly.  Pass <true> writes per-block counts; the scan
// turns them into per-block bases; pass <false> writes the positions.
// ---------------------------------------------------------------------------
// The expert ids of one chunk of CH pairs starting at p0, for one wave:
// ev[i] = id of pair p0 + 64i + lane, or -1 past the end.  Loaded once, all
// in flight together, and used by both passes.
template <int CH = kPermChunk>
__device__ __forceinline__ void load_chunk_ids(int P, int p0, int lane, const int32_t* __restrict__ ids,
                                               int (&ev)[CH / 64])
{
#pragma unroll
    for (int i = 0; i < CH / 64; i++) {
        const int p = p0 + 64 * i + lane;
        ev[i] = p < P ? ids[p] : -1;
    }
}

// Bits of an expert-id key: ids are < E and E itself marks an invalid pair.
__device__ __forceinline__ int id_key_bits(int E) { return 32 - __clz(E); }

// One wave over one chunk of CH pairs starting at p0, in pair order.
// cnt[E] (LDS) holds the chunk's running per-expert counts (zero on entry).
// A pair's rank among the equal-expert pairs of its 64 is found by ballots
// over the bits of the expert id.  Count pass: cnt ends as the chunk's
// histogram.  Position pass: pair p goes to row[e] + (earlier pairs of e in
// the chunk), row[e] being the chunk's base for expert e.
template <bool kCount, int CH = kPermChunk>
__device__ __forceinline__ void perm_chunk(int p0, int lane, int E, const int (&ev)[CH / 64],
                                           int32_t* cnt, const int32_t* row,
                                           int32_t* __restrict__ sorted_pair, int32_t* __restrict__ pair_pos)
{
    const uint64_t lower = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int nbits = id_key_bits(E);
#pragma unroll
    for (int i = 0; i < CH / 64; i++) {
        const int p = p0 + 64 * i + lane;
        const bool valid = ev[i] >= 0;
        const int e = valid ? ev[i] : 0;
        const uint32_t key = valid ? (uint32_t)e : (uint32_t)E;
        uint64_t peers = ~0ull;
        for (int bit = 0; bit < nbits; bit++) {
            const bool bb = (key >> bit) & 1u;
            const uint64_t m = __ballot(bb);
            peers &= bb ? m : ~m;
        }
        const int rank = __popcll(peers & lower);
        const int tot = __popcll(peers);
        const int base = valid ? cnt[e] : 0;
        if (!kCount && valid) {
            const int pos = row[e] + base + rank;
            sorted_pair[pos] = p;
            pair_pos[p] = pos;
        }
        __builtin_amdgcn_wave_barrier();
        if (valid && rank == tot - 1) cnt[e] = base + tot;
        __builtin_amdgcn_wave_barrier();
    }
}

// Chunk b = blockIdx.x: histogram (kCount) or positions from the per-chunk
// bases that k_perm_scan wrote over the histograms.
template <bool kCount>
__global__ __launch_bounds__(64) void k_perm_pass(int P, int E, const int32_t* __restrict__ ids,
                                                  int32_t* __restrict__ hist,
                                                  int32_t* __restrict__ sorted_pair,
                                                  int32_t* __restrict__ pair_pos)
{
    extern __shared__ int32_t cnt[];  // [E]
    const int lane = threadIdx.x;
    const int b = blockIdx.x;
    int32_t* row = hist + (size_t)b * E;
    for (int e = lane; e < E; e += 64) cnt[e] = 0;
    __syncthreads();
    int ev[kPermChunk / 64];
    load_chunk_ids(P, b * kPermChunk, lane, ids, ev);
    perm_chunk<kCount>(b * kPermChunk, lane, E, ev, cnt, row, sorted_pair, pair_pos);
    if (kCount) {
        __syncthreads();
        for (int e = lane; e < E; e += 64) row[e] = cnt[e];
    }
}

// Exclusive prefix sum of one int per thread over a 1024-thread block (wave
// scans, then a scan of the 16 wave totals).  Returns the prefix; *total gets
// the sum.  Every thread must call it.
__device__ __forceinline__ int block_exclusive_scan(int v, int* total)
{
    __shared__ int wsum[16];
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wid] = x;
    __syncthreads();
    if (wid == 0) {
        int s = lane < 16 ? wsum[lane] : 0;
        const int orig = s;
#pragma unroll
        for (int off = 1; off < 16; off <<= 1) {
            const int y = __shfl_up(s, off);
            if (lane >= off) s += y;
        }
        if (lane < 16) wsum[lane] = s - orig;
        if (lane == 15) *total = s;
    }
    __syncthreads();
    const int r = x - v + wsum[wid];
    __syncthreads();
    return r;
}

// One block: expert totals, offsets[E+1] (exclusive scan), and per-block bases
// (offsets[e] + counts of earlier blocks) written back over the counts.  The
// blocks of a column are split into P contiguous parts summed in parallel.
__global__ __launch_bounds__(1024) void k_perm_scan(int E, int nblk, int32_t* __restrict__ hist,
                                                    int32_t* __restrict__ offsets)
{
    __shared__ int32_t part_sum[1024];
    __shared__ int total_s;
    const int tid = threadIdx.x;
    const int P = max(1, min(1024 / E, nblk));
    const int e = tid % E, part = tid / E;
    const bool active = part < P;
    const int b0 = active ? (int)((long long)part * nblk / P) : 0;
    const int b1 = active ? (int)((long long)(part + 1) * nblk / P) : 0;
    // 16 loads in flight per batch (integer sums: any order gives the same total)
    constexpr int U = 16;
    int s = 0;
    for (int b = b0; b < b1; b += U) {
        int v[U];
#pragma unroll
        for (int u = 0; u < U; u++) v[u] = b + u < b1 ? hist[(size_t)(b + u) * E + e] : 0;
#pragma unroll
        for (int u = 0; u < U; u++) s += v[u];
    }
    part_sum[tid] = active ? s : 0;
    __syncthreads();
    int tot = 0;
    if (tid < E)
        for (int p = 0; p < P; p++) tot += part_sum[p * E + tid];
    int total = 0;
    const int off = block_exclusive_scan(tid < E ? tot : 0, &total_s);
    total = total_s;
    if (tid < E) offsets[tid] = off;
    if (tid == 0) offsets[E] = total;
    __syncthreads();
    // part base = offsets[e] + sums of the earlier parts of the column
    if (active) {
        int run = 0;
        for (int p = 0; p < part; p++) run += part_sum[p * E + e];
        run += offsets[e];
        for (int b = b0; b < b1; b += U) {
            int v[U];
#pragma unroll
            for (int u = 0; u < U; u++) v[u] = b + u < b1 ? hist[(size_t)(b + u) * E + e] : 0;
#pragma unroll
            for (int u = 0; u < U; u++)
                if (b + u < b1) {
                    hist[(size_t)(b + u) * E + e] = run;
                    run += v[u];
                }
        }
    }
}

// The whole permutation in one 1024-thread block when there are at most 16
// chunks of CH pairs (wave w handles chunk w): histograms, offsets and
// per-chunk bases, positions.  Same results as the three kernels above (the
// positions are the stable order whatever the chunking).  Small batches use
// 64-pair chunks, so all 16 waves share the ballot passes.  LDS:
// hist[nblk][E] then cnt[nblk][E]; off_lds (E+1 ints, optional) receives the
// offsets too.
template <int CH>
__device__ __forceinline__ void perm_small_block(int P, int E, const int32_t* __restrict__ ids,
                                                 int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
                                                 int32_t* __restrict__ pair_pos, int32_t* sh, int32_t* off_lds)
{
    __shared__ int total_s;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int nblk = (P + CH - 1) / CH;
    int32_t* hist = sh;
    int32_t* cnt = sh + nblk * E;
    int ev[CH / 64];
    if (w < nblk) load_chunk_ids<CH>(P, w * CH, lane, ids, ev);
    for (int i = tid; i < 2 * nblk * E; i += 1024) sh[i] = 0;
    __syncthreads();
    if (w < nblk) perm_chunk<true, CH>(w * CH, lane, E, ev, hist + w * E, nullptr, sorted_pair, pair_pos);
    __syncthreads();
    int tot = 0;
    if (tid < E)
        for (int b = 0; b < nblk; b++) tot += hist[b * E + tid];
    const int off = block_exclusive_scan(tid < E ? tot : 0, &total_s);
    if (tid < E) {
        offsets[tid] = off;
        if (off_lds) off_lds[tid] = off;
        int run = off;
        for (int b = 0; b < nblk; b++) {
            const int c = hist[b * E + tid];
            hist[b * E + tid] = run;
            run += c;
        }
    }
    if (tid == 0) {
        offsets[E] = total_s;
        if (off_lds) off_lds[E] = total_s;
    }
    __syncthreads();
    if (w < nblk) perm_chunk<false, CH>(w * CH, lane, E, ev, cnt + w * E, hist + w * E, sorted_pair, pair_pos);
}
template <int CH>
__global__ __launch_bounds__(1024) void k_perm_small(int P, int E, const int32_t* __restrict__ ids,
                                                     int32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ sorted_pair,
                                                     int32_t* __restrict__ pair_pos)
{
    extern __shared__ int32_t sh[];
    perm_small_block<CH>(P, E, ids, offsets, sorted_pair, pair_pos, sh, nullptr);
}

// ---------------------------------------------------------------------------
// m-tile list and persistent work queue.
// m-tile = up to M = 16*MT consecutive sorted rows of one expert.  The queue
// is ordered by scheduling waves of kWaveExperts experts (P1 §1.2, Fig. 5):
// linear1 of waves 0..D-1, then for w >= D linear1 of wave w followed by
// linear2 of wave w-D, then linear2 of the last D waves.  The lag D is chosen
// by the host so that the linear1 tiles of a wave have been taken by running
// blocks well before its linear2 tiles are, so linear2 rarely waits.  Entry =
// phase<<31 | mtile<<8 | n-block.  Also clears the persistent kernel's counters.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void build_tiles_block(int E, int M, int NB1, int NB2, int build_queue, int D,
                                                  const int32_t* offsets,
                                                  int32_t* __restrict__ mt_expert, int32_t* __restrict__ mt_row0,
                                                  int32_t* __restrict__ ctrl, int32_t* __restrict__ done1,
                                                  uint32_t* __restrict__ queue)
{
    __shared__ int32_t base[1025];
    __shared__ int32_t qstart[257];   // start of queue segment i (queue order), then the end
    __shared__ int32_t qkey[256];     // 2*wave + phase of segment i
    __shared__ int total_s, qlen_s;
    const int tid = threadIdx.x;
    const int n = tid < E ? (offsets[tid + 1] - offsets[tid] + M - 1) / M : 0;
    const int my_base = block_exclusive_scan(n, &total_s);
    base[tid] = my_base;
    if (tid == 0) base[E] = total_s;
    __syncthreads();
    const int total = base[E];
    for (int m = 0; m < n; m++) {
        mt_expert[my_base + m] = tid;
        mt_row0[my_base + m] = offsets[tid] + m * M;
    }
    for (int i = tid; i < total; i += 1024) done1[i] = 0;
    const int W = (E + kWaveExperts - 1) / kWaveExperts;
    D = max(1, min(D, W));
    // Segment order: linear1 of wave i for i < D; then, for step s = D..W-1,
    // linear1 of wave s and linear2 of wave s-D; then linear2 of waves W-D..W-1.
    // Segment index i in 0..2W-1 -> (phase, wave).
    int len = 0, ph = 0, wv = 0;
    if (build_queue == 1 && tid < 2 * W) {
        const int i = tid;
        if (i < D) { ph = 0; wv = i; }
        else if (i < 2 * W - D) { const int s2 = i - D; ph = s2 & 1; wv = ph ? (D + s2 / 2) - D : D + s2 / 2; }
        else { ph = 1; wv = W - D + (i - (2 * W - D)); }
        const int a = base[min(E, (wv + 1) * kWaveExperts)] - base[wv * kWaveExperts];
        len = a * (ph ? NB2 : NB1);
    }
    const int start = block_exclusive_scan(len, &qlen_s);
    if (build_queue == 1 && tid < 2 * W) {
        qstart[tid] = start;
        qkey[tid] = 2 * wv + ph;
    }
    if (tid == 0) {
        qstart[2 * W] = total * (NB1 + NB2);
        ctrl[0] = total;
        ctrl[1] = 0;
        ctrl[2] = build_queue == 1 ? total * (NB1 + NB2) : 0;
    }
    if (build_queue == 2) {
        // Per-XCD tile lists for the two-launch FFN: the m-tiles, in expert
        // order, cut into eight contiguous ranges of equal length (+-1); range
        // x = m-tiles ctrl[16+x] .. + ctrl[24+x] runs on XCD x (the blocks b
        // with b % 8 == x).  Its tiles are listed with each expert's column
        // blocks outer and that expert's m-tiles (within the range) inner, so
        // the tiles that read the same weights are dispatched next to each
        // other on one XCD and share its L2, and the column blocks of an
        // m-tile (the same activation rows) follow closely; a hot expert's
        // m-tiles spread over as many XCDs as their count needs.  Linear1
        // list: queue[s0*NB1 ..]; linear2 list: queue[ctrl[4] + s0*NB2 ..];
        // entry = m-tile<<8 | column block.
        if (tid < 8) {
            const int s0 = (int)((long long)tid * total / 8), s1 = (int)((long long)(tid + 1) * total / 8);
            ctrl[16 + tid] = s0;
            ctrl[24 + tid] = s1 - s0;
        }
        if (tid == 0) ctrl[4] = total * NB1;
        if (n > 0) {
            for (int x = 0; x < 8; x++) {
                const int s0 = (int)((long long)x * total / 8), s1 = (int)((long long)(x + 1) * total / 8);
                const int g0 = max(my_base, s0), g1 = min(my_base + n, s1), gl = g1 - g0;
                for (int i = g0; i < g1; i++) {
                    for (int nb = 0; nb < NB1; nb++)
                        queue[(size_t)g0 * NB1 + nb * gl + (i - g0)] = ((uint32_t)i << 8) | (uint32_t)nb;
                    for (int nb = 0; nb < NB2; nb++)
                        queue[(size_t)total * NB1 + (size_t)g0 * NB2 + nb * gl + (i - g0)] =
                            ((uint32_t)i << 8) | (uint32_t)nb;
                }
            }
        }
        return;
    }
    if (build_queue != 1) return;
    __syncthreads();
    // segments to waves in turn, a segment's entries to the wave's lanes
    const int qw = tid >> 6, ln = tid & 63;
    for (int sg = qw; sg < 2 * W; sg += 16) {
        const int q0 = qstart[sg], len = qstart[sg + 1] - q0;
        const int swv = qkey[sg] >> 1, sph = qkey[sg] & 1;
        const int NB = sph ? NB2 : NB1;
        const int mt0 = base[swv * kWaveExperts];
        for (int i = ln; i < len; i += 64)
            queue[q0 + i] = ((uint32_t)sph << 31) | ((uint32_t)(mt0 + i / NB) << 8) | (uint32_t)(i % NB);
    }
}
__global__ __launch_bounds__(1024) void k_build_tiles(int E, int M, int NB1, int NB2, int build_queue, int D,
                                                      const int32_t* __restrict__ offsets,
                                                      int32_t* __restrict__ mt_expert,
                                                      int32_t* __restrict__ mt_row0,
                                                      int32_t* __restrict__ ctrl,
                                                      int32_t* __restrict__ done1,
                                                      uint32_t* __restrict__ queue)
{
    build_tiles_block(E, M, NB1, NB2, build_queue, D, offsets, mt_expert, mt_row0, ctrl, done1, queue);
}

// Small batches: the permutation and the m-tile list / work queue in one
// 1024-thread block, the same device code as k_perm_small and k_build_tiles
// run one after the other (the tile list reads the offsets after a block
// barrier), so the results are identical; one dependent launch fewer on the
// latency-bound path.
template <int CH>
__global__ __launch_bounds__(1024) void k_perm_tiles(int P, int E, const int32_t* __restrict__ ids,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ sorted_pair,
                                                     int32_t* __restrict__ pair_pos, int M, int NB1, int NB2,
                                                     int build_queue, int D, int32_t* __restrict__ mt_expert,
                                                     int32_t* __restrict__ mt_row0, int32_t* __restrict__ ctrl,
                                                     int32_t* __restrict__ done1, uint32_t* __restrict__ queue)
{
    extern __shared__ int32_t sh[];
    __shared__ int32_t off_lds[1025];
    perm_small_block<CH>(P, E, ids, offsets, sorted_pair, pair_pos, sh, off_lds);
    __syncthreads();
    // the tile list reads the offsets from LDS, not back from global memory
    build_tiles_block(E, M, NB1, NB2, build_queue, D, off_lds, mt_expert, mt_row0, ctrl, done1, queue);
}

// ---------------------------------------------------------------------------
// Expert FFN tiles.
//
// A tile is one m-tile (M = 16*MT rows of one expert) by a block of output
// columns, computed by NW = RW*CW waves: RW row groups of MTW = MT/RW m-tiles
// each, and CW column groups.  Wave w = (rg, cg) = (w / CW, w % CW) owns eight
// 16-column n-tiles of its row group:
//   phase 1 (linear1 + SwiGLU + requant, K = H): gate n-tiles 4cg..4cg+3 and
//     the up n-tiles of the same columns of the tile's HC = 64*CW columns of
//     h, so both halves of a SwiGLU pair sit in one lane;
//   phase 2 (linear2, K = I): output n-tiles 8cg..8cg+7 of OC = 128*CW columns.
//
// Data movement: an NS-stage ring in LDS, one stage per 128-wide K chunk,
// filled NS-1 chunks ahead by gfx950 direct-to-LDS loads (global_load_lds):
//   B  the tile's 8*CW packed FP4 records (1 KiB each, contiguous in HBM) and
//      2*CW E8M0 records (256 B: one dword per lane = the scale bytes of four
//      n-tiles), 16 / 4 bytes per lane, fully coalesced;
//   A  the tile's M activation rows (E4M3, 128 B per chunk), gathered through
//      sorted_pair in phase 1, contiguous hq rows in phase 2.  Lanes write LDS
//      contiguously, so each row's 16-byte segments are stored XOR-swizzled by
//      (row/2)%8, which puts the 16 rows of one operand read on distinct banks;
//   X  the per-row activation scales of the chunk, token-major (a lane reads
//      its token's scales for all its token tiles at once).
// Stages are consumed in order: wait for the stage's loads (s_waitcnt vmcnt,
// counted per wave), one barrier, issue the loads NS-1 chunks ahead into the
// slot just freed, compute: per 16-token tile, eight block-scaled MFMAs with
// the weights as the A operand (FP4 codes and their E8M0 scales straight from
// LDS, no dequantisation pass) and the tokens as the B operand, so a lane gets
// four consecutive output columns of one token; then acc = fma(xs*blk, P, acc)
// with one activation scale per token tile.  A 16-token tile with no valid
// row skips its MFMAs.
// ---------------------------------------------------------------------------

// Stores that another XCD may read within the same launch: agent-scope
// (relaxed) atomic stores, which on gfx950 write through the local L2.
__device__ __forceinline__ void store_coherent(float* p, float v)
{
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_coherent(uint8_t* p, uint4 v);
// h and its scales: agent-coherent stores when linear2 tiles of the same launch
// read them (the persistent kernel), plain stores when the next launch does.
template <bool COH>
__device__ __forceinline__ void store_h(float* p, float v)
{
    if (COH) store_coherent(p, v);
    else *p = v;
}
template <bool COH>
__device__ __forceinline__ void store_h(uint8_t* p, uint4 v)
{
    if (COH) store_coherent(p, v);
    else *reinterpret_cast<uint4*>(p) = v;
}
__device__ __forceinline__ void store_coherent(uint8_t* p, uint4 v)
{
    uint64_t* q = reinterpret_cast<uint64_t*>(p);
    __hip_atomic_store(q, (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(q + 1, (uint64_t)v.z | ((uint64_t)v.w << 32), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Direct-to-LDS copies: each lane moves 16 (or 4) bytes from its own global
// address to lds_base + lane*16 (lane*4); lds_base is wave-uniform (M0).  As
// inline asm they are invisible to the compiler's wait insertion, which would
// otherwise drain the whole pipeline before every LDS read; completion is
// awaited explicitly with wait_vm<N>() (at most N of this wave's vector memory
// operations still outstanding).  The global address is a wave-uniform 64-bit
// base (SGPRs) plus a 32-bit per-lane byte offset.
__device__ __forceinline__ void dma16s(const void* base, uint32_t off, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
__device__ __forceinline__ void dma4s(const void* base, uint32_t off, uint32_t lds_base)
{
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
                 :: "v"(off), "s"(base), "s"(lds_base) : "memory", "m0");
}
// wait until at most OPS*k operations are outstanding, k = 0..2 at run time
template <int OPS>
__device__ __forceinline__ void wait_stages(int k)
{
    if (k >= 2) wait_vm<2 * OPS>();
    else if (k == 1) wait_vm<OPS>();
    else wait_vm<0>();
}

// Ring depth: 128-row m-tiles with two wave columns keep two stages, so that
// two blocks share a CU (each block's per-chunk barrier and operand reads
// then overlap the other's MFMAs).
__host__ __device__ constexpr int ring_stages(int MT, int CW) { return MT == 1 ? 4 : (MT == 8 && CW == 2 ? 2 : 3); }

template <int MT, int RW, int CW>
struct TileLayout {
    static constexpr int NW = RW * CW;
    static constexpr int NT = 64 * NW;                       // threads
    static constexpr int M = 16 * MT;
    static constexpr int MTW = MT / RW;                      // m-tiles per wave
    static constexpr int RG = M / RW;                        // rows per row group
    static constexpr int HC = 64 * CW;                       // phase-1 columns of h
    static constexpr int OC = 128 * CW;                      // phase-2 output columns
    static constexpr int NS = ring_stages(MT, CW);
    static constexpr int NBR = 8 / RW;                       // B records per wave per stage
    static constexpr int NSR = 2 / RW;                       // scale records per wave per stage
    static constexpr int AB = M / 8;                         // 1 KiB A blocks per stage
    static constexpr int AI = AB >= NW ? AB / NW : 1;        // A loads per wave per stage
    static constexpr int OPS = NBR + NSR + AI + 1;           // loads per wave per stage
    static constexpr int B_OFF = 0;                          // 8*CW records x 1 KiB
    static constexpr int S_OFF = 8 * CW * 1024;              // 2*CW records x 256 B
    static constexpr int A_OFF = S_OFF + 2 * CW * 256;       // M rows x 128 B (swizzled)
    static constexpr int X_OFF = A_OFF + M * 128;            // RW x 64 floats
    static constexpr int STAGE = X_OFF + RW * 256;
    static constexpr int RING = NS * STAGE;
    static constexpr int ROW_OFF = RING;                     // [M] int
    static constexpr int BLK_OFF = ROW_OFF + M * 4;          // [CW][128] float: block scales per chunk
    static constexpr int BYTES = BLK_OFF + CW * 128 * 4;
    static constexpr int SP1 = HC + 16;                      // phase-1 staging pitch (bytes)
    static constexpr int SP2 = OC + 8;                       // phase-2 staging pitch (bf16)
    static_assert(MT % RW == 0 && RG <= 64, "a row group's scales fit one 64-lane load");
    static_assert(CW == 2 || CW == 4, "a 128-column quantisation group spans two waves");
    static_assert(RW == 1 || RW == 2, "");
    static_assert(AB % NW == 0 || NW % AB == 0, "A blocks spread evenly over the waves");
    static_assert(OPS * (NS - 2) < 64, "vmcnt range");
    static_assert(NS >= 2 && STAGE >= M * SP1 && STAGE >= NW * RG * 4 && STAGE >= RW * 16 * SP2 * 2,
                  "epilogue staging and amax partials fit in a stage");
};

// SiLU(g) * u in fp32 (the same code in every tile variant).
__device__ __forceinline__ float swiglu(float g, float u) { return (g / (1.0f + expf(-g))) * u; }

// Gate-less activations (the cheap alternative to SwiGLU): squared ReLU, or
// ReLU; both need neither an exponential nor a division.
__device__ __forceinline__ float gateless_act(int act, float u)
{
    const float r = u > 0.0f ? u : 0.0f;
    return act == 1 ? r * r : r;
}

// Optional export of the linear1 outputs before the activation (fp32, sorted
// rows; the backward recomputes them this way): lane l of a wave holds, for
// the token l%16 of each token tile i, four consecutive columns
// col0 + 16j + 4(l/16) .. +3 in acc[i][j0 + j], j < NJ.
template <int MTW>
__device__ __forceinline__ void store_linear1(float* out, const FfnArgs& a, int row0, int rows, int rbase, int col0,
                                              const v4f (&acc)[MTW][8], int j0, int nj = 8)
{
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < MTW; i++) {
        const int r = rbase + i * 16 + (lane & 15);
        if (r >= rows) continue;
        float* dst = out + (size_t)(row0 + r) * a.I + col0 + 4 * (lane >> 4);
#pragma unroll
        for (int j = 0; j < 8; j++)
            if (j < nj)
                *reinterpret_cast<float4*>(dst + 16 * j) =
                    make_float4(acc[i][j0 + j][0], acc[i][j0 + j][1], acc[i][j0 + j][2], acc[i][j0 + j][3]);
    }
}

// G: the expert FFN is SwiGLU (gate and up projections); otherwise gate-less
// (a.act selects the activation).  Phase 2 does not depend on G.
template <int PHASE, int MT, int RW, int CW, bool G, bool COH = true>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int mt, int nb, uint8_t* smem)
{
    using TL = TileLayout<MT, RW, CW>;
    constexpr int M = TL::M, NS = TL::NS, NT = TL::NT, NW = TL::NW, MTW = TL::MTW, RG = TL::RG;
    // columns of h per linear1 tile: gated, each wave's eight n-tiles pair 64
    // gate with 64 up columns; gate-less, they are 128 columns of h
    constexpr int HC1 = G ? TL::HC : 2 * TL::HC;
    constexpr int SP1 = HC1 + 16;                            // phase-1 staging pitch (bytes)
    static_assert(M * SP1 <= TL::RING, "phase-1 staging fits the ring");
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int rg = w / CW, cg = w % CW;
    const int e = uniform(a.mt_expert[mt]);
    const int row0 = uniform(a.mt_row0[mt]);
    const int rows = uniform(min(M, a.offsets[e + 1] - row0));
    const bool active = rows > rg * RG;                      // this row group has a valid row
    const int nti = uniform(min(MTW, (rows - rg * RG + 15) / 16));  // token tiles with a valid row
    const int K = PHASE == 1 ? a.H : a.I;
    const int N = PHASE == 1 ? a.I : a.H;
    const int C = K / 128;
    const uint32_t ring = (uint32_t)(uintptr_t)smem;

    int32_t* rowinfo = reinterpret_cast<int32_t*>(smem + TL::ROW_OFF);

    // phase 1: token of each row (rows past the end repeat the last valid
    // row's token: finite filler, never stored); phase 2: pair id or -1.
    for (int r = tid; r < M; r += NT) {
        const int p = a.sorted_pair[row0 + min(r, rows - 1)];
        rowinfo[r] = PHASE == 1 ? p / a.topk : (r < rows ? p : -1);
    }
    // The tile's 128x128 block scales for every chunk, staged in LDS (per-chunk
    // global reads would be vector loads whose waits drain the load ring).
    // Phase 1 gated: [2*hb] gate, [2*hb+1] up of h block hb of the tile;
    // otherwise: output block cg of the tile (linear1 gate-less, linear2).
    float* blkv = reinterpret_cast<float*>(smem + TL::BLK_OFF);
    for (int i = tid; i < CW * C; i += NT) {
        const int h = i / C, c = i % C;
        const float* src = PHASE == 1
            ? (G ? ((h & 1) ? a.up.blk : a.gate.blk) + ((size_t)e * (a.I / 128) + nb * (CW / 2) + (h >> 1)) * C
                 : a.up.blk + ((size_t)e * (a.I / 128) + nb * CW + h) * C)
            : a.down.blk + ((size_t)e * (a.H / 128) + nb * CW + h) * C;
        blkv[h * 128 + c] = src[c];
    }
    __syncthreads();

    // Sources of this wave's loads at chunk 0: wave-uniform bases plus 32-bit
    // per-lane byte offsets (the dimension checks keep every offset < 2^31).
    const uint8_t* bbase[TL::NBR];
#pragma unroll
    for (int r = 0; r < TL::NBR; r++) {
        const int rr = w * TL::NBR + r;                      // record of the tile, 0 .. 8*CW-1
        const MatPtr& m = PHASE == 1 ? (G && (rr & 7) < 4 ? a.gate : a.up) : a.down;
        const int tile = PHASE == 1 && G ? nb * 4 * CW + 4 * (rr >> 3) + (rr & 3) : nb * 8 * CW + rr;
        bbase[r] = uniform(m.fp4 + ((size_t)e * (N / 16) + tile) * C * 1024);
    }
    const uint8_t* sbase[TL::NSR];
#pragma unroll
    for (int r = 0; r < TL::NSR; r++) {
        const int ss = w * TL::NSR + r;                      // scale record, 0 .. 2*CW-1
        const MatPtr& m = PHASE == 1 ? (G && (ss & 1) == 0 ? a.gate : a.up) : a.down;
        const int quad = PHASE == 1 && G ? nb * CW + (ss >> 1) : nb * 2 * CW + ss;
        sbase[r] = uniform(m.e8m0 + ((size_t)e * (N / 64) + quad) * C * 256);
    }
    const float* blk0 = blkv + (PHASE == 1 && G ? 2 * (cg >> 1) : cg) * 128;
    const float* blk1 = blkv + (PHASE == 1 && G ? 2 * (cg >> 1) + 1 : cg) * 128;
    const uint8_t* abase = uniform(PHASE == 1 ? a.xq : a.hq);
    uint32_t aoff[TL::AI];
#pragma unroll
    for (int i = 0; i < TL::AI; i++) {
        const int blk = (i * NW + w) % TL::AB;               // 1 KiB block = 8 rows
        const int g = blk * 64 + lane;                       // 16-byte segment of the tile
        const int r = g >> 3;
        const int seg = (g & 7) ^ ((r >> 1) & 7);            // global segment stored at position g&7
        const int rc = min(r, rows - 1);
        aoff[i] = (PHASE == 1 ? (uint32_t)rowinfo[r] * (uint32_t)a.H : (uint32_t)(row0 + rc) * (uint32_t)a.I) +
                  seg * 16;
    }
    const float* xbase = uniform(PHASE == 1 ? a.xs : a.hs);
    // activation scales of the row group, stored token-major: position
    // t*MTW + i holds row i*16 + t, so a lane reads the scales of its token in
    // all MTW token tiles with one LDS read
    uint32_t xoff;
    {
        const int p = min(lane, RG - 1);
        const int r = min(rg * RG + (p % MTW) * 16 + p / MTW, M - 1);
        xoff = 4u * (PHASE == 1 ? (uint32_t)rowinfo[r] * (uint32_t)(a.H / 128)
                                : (uint32_t)(row0 + min(r, rows - 1)) * (uint32_t)a.hs_stride);
    }

    auto issue = [&](int c, int slot) {
        const uint32_t st = __builtin_amdgcn_readfirstlane(ring + slot * TL::STAGE);
#pragma unroll
        for (int r = 0; r < TL::NBR; r++)
            dma16s(bbase[r], lane * 16 + c * 1024, st + TL::B_OFF + (w * TL::NBR + r) * 1024);
#pragma unroll
        for (int r = 0; r < TL::NSR; r++)
            dma4s(sbase[r], lane * 4 + c * 256, st + TL::S_OFF + (w * TL::NSR + r) * 256);
#pragma unroll
        for (int i = 0; i < TL::AI; i++)
            dma16s(abase, aoff[i] + c * 128, st + TL::A_OFF + ((i * NW + w) % TL::AB) * 1024);
        dma4s(xbase, xoff + c * 4, st + TL::X_OFF + rg * 256);
    };

    v4f acc[MTW][8];
#pragma unroll
    for (int i = 0; i < MTW; i++)
#pragma unroll
        for (int j = 0; j < 8; j++) acc[i][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

#pragma unroll
    for (int u = 0; u < NS - 1; u++)
        if (u < C) issue(u, u);

    // The chunk loop is instantiated per count of token tiles holding a valid
    // row, chosen once per wave (only the last m-tile of an expert has fewer
    // than MTW).  Every instance runs the same sequence of barriers, one per
    // chunk, so waves of different row groups may run different instances.
    auto chunk_loop = [&](auto count) {
        constexpr int NTI = decltype(count)::value;
        for (int c = 0; c < C; c++) {
            wait_stages<TL::OPS>(min(NS - 2, C - 1 - c));
            __syncthreads();
            if (c + NS - 1 < C) issue(c + NS - 1, (c + NS - 1) % NS);
            if (!active) continue;

            const uint8_t* st = smem + (c % NS) * TL::STAGE;
            uint4 bq[8];
#pragma unroll
            for (int j = 0; j < 8; j++)
                bq[j] = *reinterpret_cast<const uint4*>(st + TL::B_OFF + (cg * 8 + j) * 1024 + lane * 16);
            const int sc[2] = {*reinterpret_cast<const int*>(st + TL::S_OFF + (cg * 2) * 256 + lane * 4),
                               *reinterpret_cast<const int*>(st + TL::S_OFF + (cg * 2 + 1) * 256 + lane * 4)};
            const float sb0 = blk0[c];
            const float sb1 = blk1[c];
            // this lane's token in each token tile: one activation scale per tile
            float xsv[MTW];
            {
                const float* xr = reinterpret_cast<const float*>(st + TL::X_OFF + rg * 256) + (lane & 15) * MTW;
                if (MTW == 4) {
                    const float4 v = *reinterpret_cast<const float4*>(xr);
                    xsv[0] = v.x; xsv[1] = v.y; xsv[2 % MTW] = v.z; xsv[3 % MTW] = v.w;
                } else if (MTW == 2) {
                    const float2 v = *reinterpret_cast<const float2*>(xr);
                    xsv[0] = v.x; xsv[1 % MTW] = v.y;
                } else {
#pragma unroll
                    for (int i = 0; i < MTW; i++) xsv[i] = xr[i];
                }
            }
            // Every token tile with a valid row is computed (rows past the end
            // hold finite filler and are never stored; tiles wholly past the end
            // keep zero accumulators), in straight-line code: the eight
            // independent MFMAs of a token tile are all in flight before their
            // results are promoted.
#pragma unroll
            for (int i = 0; i < NTI; i++) {
                const int r = rg * RG + i * 16 + (lane & 15);
                const int sw = (r >> 1) & 7;
                const int g = lane >> 4;
                const uint8_t* arow = st + TL::A_OFF + r * 128;
                const uint4 a0 = *reinterpret_cast<const uint4*>(arow + ((g ^ sw) * 16));
                const uint4 a1 = *reinterpret_cast<const uint4*>(arow + (((g + 4) ^ sw) * 16));
                const v8i xf = {(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                                (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
                v4f P[8];
#pragma unroll
                for (int j = 0; j < 8; j++) P[j] = mfma_e2m1_e4m3_sel(j & 3, bq[j], sc[j >> 2], xf);
                const float s0 = xsv[i] * sb0;
                const float s1 = xsv[i] * sb1;
#pragma unroll
                for (int j = 0; j < 8; j++) {
                    const float s = (PHASE == 1 && G && j >= 4) ? s1 : s0;
#pragma unroll
                    for (int q = 0; q < 4; q++) acc[i][j][q] = __builtin_fmaf(s, P[j][q], acc[i][j][q]);
                }
            }
        }
    };
    if (nti >= MTW) chunk_loop(std::integral_constant<int, MTW>{});
    else if (MTW >= 4 && nti == 3) chunk_loop(std::integral_constant<int, (MTW >= 4 ? 3 : 1)>{});
    else if (MTW >= 2 && nti == 2) chunk_loop(std::integral_constant<int, (MTW >= 2 ? 2 : 1)>{});
    else chunk_loop(std::integral_constant<int, 1>{});
    __syncthreads();   // every wave is done with the ring: its first stages become staging space

    if (PHASE == 1 && !G) {
        // h = act(u), then E4M3 per (row, 128 columns of h).  Lane l holds, for
        // the token l%16 of each token tile, h columns 128cg + 16j + 4(l/16) + q
        // (j < 8, q < 4): one wave owns a whole 128-column group, so the row
        // amax is reduced over the lane's 32 values and the four lanes of the
        // token (xor 16, 32).
        uint8_t* stage = smem;                                      // [M][SP1]
        const int g = lane >> 4;
        const int act = a.act;
        if (a.u_out) store_linear1(a.u_out, a, row0, rows, rg * RG, nb * HC1 + 128 * cg, acc, 0);
#pragma unroll
        for (int i = 0; i < MTW; i++) {
            float mx = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    acc[i][j][q] = gateless_act(act, acc[i][j][q]);
                    mx = fmaxf(mx, acc[i][j][q]);                   // h >= 0
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            const int r = rg * RG + i * 16 + (lane & 15);
            const float s = mx > 0.0f ? mx / 448.0f : 1.0f;
            const float inv = 1.0f / s;
            if (g == 0 && r < rows)
                store_h<COH>(a.hs + (size_t)(row0 + r) * a.hs_stride + nb * CW + cg, s);
#pragma unroll
            for (int j = 0; j < 8; j++)
                *reinterpret_cast<uint32_t*>(stage + r * SP1 + 128 * cg + 16 * j + 4 * g) =
                    e4m3x2(acc[i][j][0] * inv, acc[i][j][1] * inv) |
                    (e4m3x2(acc[i][j][2] * inv, acc[i][j][3] * inv) << 16);
        }
        __syncthreads();
        constexpr int SEGS = HC1 / 16;
        for (int s = tid; s < M * SEGS; s += NT) {
            const int r = s / SEGS, sg = s % SEGS;
            if (r < rows)
                store_h<COH>(a.hq + (size_t)(row0 + r) * a.I + nb * HC1 + sg * 16,
                               *reinterpret_cast<const uint4*>(stage + r * SP1 + sg * 16));
        }
        __syncthreads();
    } else if (PHASE == 1) {
        // h = SiLU(g) * u, then E4M3 per (row, 128 columns of h).  Lane l holds,
        // for the token l%16 of each token tile, h columns 64cg + 16j + 4(l/16)
        // + q (j < 4, q < 4): the row amax is reduced over the lane's 16 values,
        // the four lanes of the token (xor 16, 32), then over the two waves
        // that share the 128 columns.
        uint8_t* stage = smem;                                      // [M][SP1]
        float* red = reinterpret_cast<float*>(smem + TL::STAGE);    // [NW][RG], ring stage 1
        const int g = lane >> 4;
        if (a.g_out) {
            store_linear1(a.g_out, a, row0, rows, rg * RG, nb * HC1 + 64 * cg, acc, 0, 4);
            store_linear1(a.u_out, a, row0, rows, rg * RG, nb * HC1 + 64 * cg, acc, 4, 4);
        }
        float hv[MTW][4][4];
#pragma unroll
        for (int i = 0; i < MTW; i++) {
            float mx = 0.0f;
#pragma unroll
            for (int j = 0; j < 4; j++)
#pragma unroll
                for (int q = 0; q < 4; q++) {
                    const float h = silu_mul(acc[i][j][q], acc[i][4 + j][q]);
                    hv[i][j][q] = h;
                    mx = fmaxf(mx, fabsf(h));
                }
            mx = fmaxf(mx, __shfl_xor(mx, 16));
            mx = fmaxf(mx, __shfl_xor(mx, 32));
            if (g == 0) red[w * RG + i * 16 + (lane & 15)] = mx;
        }
        __syncthreads();
        const int wp = rg * CW + (cg & ~1);
#pragma unroll
        for (int i = 0; i < MTW; i++) {
            const int rl = i * 16 + (lane & 15);
            const int r = rg * RG + rl;
            const float amax = fmaxf(red[wp * RG + rl], red[(wp + 1) * RG + rl]);
            const float s = amax > 0.0f ? amax / 448.0f : 1.0f;
            const float inv = 1.0f / s;
            if ((cg & 1) == 0 && g == 0 && r < rows)
                store_h<COH>(a.hs + (size_t)(row0 + r) * a.hs_stride + nb * (CW / 2) + (cg >> 1), s);
#pragma unroll
            for (int j = 0; j < 4; j++)
                *reinterpret_cast<uint32_t*>(stage + r * SP1 + 64 * cg + 16 * j + 4 * g) =
                    e4m3x2(hv[i][j][0] * inv, hv[i][j][1] * inv) | (e4m3x2(hv[i][j][2] * inv, hv[i][j][3] * inv) << 16);
        }
        __syncthreads();
        constexpr int SEGS = HC1 / 16;
        for (int s = tid; s < M * SEGS; s += NT) {
            const int r = s / SEGS, sg = s % SEGS;
            if (r < rows)
                store_h<COH>(a.hq + (size_t)(row0 + r) * a.I + nb * HC1 + sg * 16,
                               *reinterpret_cast<const uint4*>(stage + r * SP1 + sg * 16));
        }
        __syncthreads();
    } else {
        // bf16 rows scattered back to their pair slot p = t*topk + j, one m-tile
        // of every row group at a time.
        uint16_t* stage = reinterpret_cast<uint16_t*>(smem);        // [RW*16][SP2]
        constexpr int SEGS = TL::OC / 8;
#pragma unroll
        for (int i = 0; i < MTW; i++) {
            if (i * 16 < rows) {
#pragma unroll
                for (int j = 0; j < 8; j++)
                    *reinterpret_cast<uint2*>(stage + (rg * 16 + (lane & 15)) * TL::SP2 + 128 * cg + 16 * j +
                                              4 * (lane >> 4)) =
                        make_uint2(bf16x2(acc[i][j][0], acc[i][j][1]), bf16x2(acc[i][j][2], acc[i][j][3]));
                __syncthreads();
                for (int s = tid; s < RW * 16 * SEGS; s += NT) {
                    const int rs = s / SEGS, sg = s % SEGS;
                    const int r = (rs >> 4) * RG + i * 16 + (rs & 15);
                    if (r < rows) {
                        const int p = rowinfo[r];
                        *reinterpret_cast<uint4*>(a.y + (size_t)p * a.H + nb * TL::OC + sg * 8) =
                            *reinterpret_cast<const uint4*>(stage + rs * TL::SP2 + sg * 8);
                    }
                }
                __syncthreads();
            }
        }
    }
}

template <int PHASE, int MT, int RW, int CW, bool G>
__global__ __launch_bounds__(64 * RW * CW) void k_ffn(FfnArgs a, int NB)
{
    extern __shared__ __align__(16) uint8_t smem[];
    int mt, nb;
    if (a.xcd_groups) {
        // block b runs on XCD b % 8 (round-robin dispatch): entry b / 8 of
        // that XCD's tile list
        const int x = blockIdx.x & 7, j = blockIdx.x >> 3;
        if (j >= a.ctrl[24 + x] * NB) return;
        const uint32_t it = a.queue[(PHASE == 1 ? 0 : a.ctrl[4]) + a.ctrl[16 + x] * NB + j];
        mt = (int)(it >> 8);
        nb = (int)(it & 0xFFu);
    } else {
        mt = blockIdx.x / NB;
        nb = blockIdx.x % NB;
        if (mt >= a.ctrl[0]) return;
    }
    ffn_tile<PHASE, MT, RW, CW, G, false>(a, mt, nb, smem);   // the next launch reads h
}

// Persistent, wave-scheduled: blocks take queue entries in order.  A linear2
// tile waits until all linear1 tiles of its m-tile are done; those entries sit
// earlier in the queue, were taken by running blocks and never wait, so every
// wait ends.  Counters only signal readiness; no data is accumulated through
// them, so the numerics are those of the unfused kernels.
template <int MT, int RW, int CW, bool G>
__global__ __launch_bounds__(64 * RW * CW) void k_ffn_persistent(FfnArgs a)
{
    extern __shared__ __align__(16) uint8_t smem[];
    __shared__ uint32_t item;
    const int NB1 = a.I / (TileLayout<MT, RW, CW>::HC * (G ? 1 : 2));
    const int total = a.ctrl[2];
    for (;;) {
        __syncthreads();
        if (threadIdx.x == 0) {
            const int q = atomicAdd(&a.ctrl[1], 1);
            item = q < total ? a.queue[q] : 0xFFFFFFFFu;
        }
        __syncthreads();
        const uint32_t it = item;
        if (it == 0xFFFFFFFFu) break;
        const int mt = (int)((it >> 8) & 0x7FFFFFu);
        const int nb = (int)(it & 0xFFu);
        if ((it >> 31) == 0) {
            // h and its scales were written with agent-coherent stores (through
            // this XCD's L2); once every wave has them acknowledged, one counter
            // increment publishes the tile.  No L2 write-back is needed.
            ffn_tile<1, MT, RW, CW, G>(a, mt, nb, smem);
            wait_vm<0>();
            __syncthreads();
            if (threadIdx.x == 0)
                __hip_atomic_fetch_add(&a.done1[mt], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
            if (threadIdx.x == 0) {
                while (__hip_atomic_load(&a.done1[mt], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < NB1)
                    __builtin_amdgcn_s_sleep(2);
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // drop any stale cached lines
            }
            __syncthreads();
            ffn_tile<2, MT, RW, CW, G>(a, mt, nb, smem);
        }
    }
}

// ---------------------------------------------------------------------------
// Combine: out[t] = bf16(sum_j w[t][j] * y[t*k+j]) in fp32, j ascending.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(int T, int H, int k, const uint16_t* __restrict__ y,
                                                 const float* __restrict__ w, uint16_t* __restrict__ out)
{
    const size_t total = (size_t)T * H / 8;
    const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total) return;
    const size_t t = idx / (H / 8);
    const size_t c = idx % (H / 8);
    float acc[8] = {0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f, 0.0f};
    auto add = [&](float wj, uint4 v) {
        const uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int u = 0; u < 4; u++) {
            acc[2 * u] = __builtin_fmaf(wj, bf16_to_f32(q[u] & 0xFFFFu), acc[2 * u]);
            acc[2 * u + 1] = __builtin_fmaf(wj, bf16_to_f32(q[u] >> 16), acc[2 * u + 1]);
        }
    };
    // the rows of the first eight slots are all loaded before any is added,
    // then added in slot order (further slots follow in order)
    constexpr int KU = 8;
    uint4 v[KU];
    float wv[KU];
#pragma unroll
    for (int j = 0; j < KU; j++)
        if (j < k) {
            wv[j] = w[t * k + j];
            v[j] = *reinterpret_cast<const uint4*>(y + (t * k + j) * H + c * 8);
        }
#pragma unroll
    for (int j = 0; j < KU; j++)
        if (j < k) add(wv[j], v[j]);
    for (int j = KU; j < k; j++)
        add(w[t * k + j], *reinterpret_cast<const uint4*>(y + (t * k + j) * H + c * 8));
    const uint4 o = make_uint4(bf16x2(acc[0], acc[1]), bf16x2(acc[2], acc[3]), bf16x2(acc[4], acc[5]),
                               bf16x2(acc[6], acc[7]));
    *reinterpret_cast<uint4*>(out + t * H + c * 8) = o;
}

// ---------------------------------------------------------------------------
// Offline weight prepack and the dequantisation export
// ---------------------------------------------------------------------------
// Canonical -> packed.  One thread per 16-byte FP4 slot (expert, 16-row
// n-tile, 128-wide K chunk, lane): the slot's 32 codes keep the canonical
// nibble order (the matrix cores read element k from nibble k%2 of byte k/2);
// the slot's E8M0 byte goes to byte tile%4 of the lane's dword in the record
// of its n-tile quad.  Flags any scale outside the lossless window.
__global__ __launch_bounds__(256) void k_prepack(int E, int N, int K, const uint8_t* __restrict__ fin,
                                                 const uint8_t* __restrict__ ein,
                                                 uint8_t* __restrict__ fout, uint8_t* __restrict__ eout,
                                                 int32_t* __restrict__ bad)
{
    const int C = K / 128;
    const size_t total = (size_t)E * (N / 16) * C * 64;
    const size_t slot = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (slot >= total) return;
    const int lane = (int)(slot & 63);
    const size_t rec = slot >> 6;
    const int c = (int)(rec % C);
    const int tile = (int)((rec / C) % (N / 16));
    const size_t e = rec / C / (N / 16);
    const int n = tile * 16 + (lane & 15);
    const int k0 = c * 128 + (lane >> 4) * 32;
    *reinterpret_cast<uint4*>(fout + slot * 16) =
        *reinterpret_cast<const uint4*>(fin + (e * N + n) * (size_t)(K / 2) + k0 / 2);
    const uint8_t s = ein[(e * N + n) * (size_t)(K / 32) + k0 / 32];
    eout[((e * (N / 64) + tile / 4) * C + c) * 256 + lane * 4 + (tile & 3)] = s;
    if (s < 127 - 8 || s > 127 + 6) atomicOr(bad, 1);
}

// FP32 master weights -> MXFP4 under fp32 128x128 block scales (P1 §4 and
// P4 §4: the QAT forward quantises the FP32 master weights to FP4; format per
// the OCP MX paper the pages cite).  256 threads per 128x128 block; float4
// f = i*256 + tid of the block is row f/32, columns 4*(f%32)..+3, so a 1x32
// sub-block is 8 consecutive lanes.
//   s = amax / 384 (fp32; 1 for an all-zero block): the block's largest
//       magnitude lands on 6 * 2^6, FP4's largest value at the top of the
//       lossless window;
//   v = w / s (fp32); sub-block exponent b = floor(log2(max|v|)) - 2 (OCP MX
//       shared exponent, E2M1's largest exponent being 2), raised to -8 below
//       the window (counted in *clamped), 0 for an all-zero sub-block;
//   code = nearest E2M1 of v * 2^-b, ties to the even code, saturating at 6,
//       sign kept (the hardware conversion, e2m1x4).
// The max of v over each group of 8 consecutive lanes (DPP: swap neighbours,
// swap pairs, mirror the two quads of the group).
__device__ __forceinline__ float max8_lanes(float v)
{
    auto dpp = [](float x, auto ctrl) {
        return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), decltype(ctrl)::value, 0xF, 0xF, false));
    };
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0xB1>{}));    // quad_perm [1,0,3,2]
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x4E>{}));    // quad_perm [2,3,0,1]
    v = fmaxf(v, dpp(v, std::integral_constant<int, 0x141>{}));   // row_half_mirror
    return v;
}

// LDS staging pitch of the code rows (128 bytes of codes + 16: the 16-byte
// reads of the packed copy-out, 16 rows apart, fall on distinct banks).
constexpr int kQuantPitch = 144;

// One 128x128 block: rows r = 8i + tid/32 (i < 16) held as float4 v[i]; the
// codes (2 bytes per lane per row) and sub-block exponents go to LDS staging
// rows (f4s: kQuantPitch bytes per row, e8s: 8 bytes per row) at column
// offset h of the block pair.
// FAST: v = w/s as RN(w * y) with y = RN(1/s), then two residual corrections
// r = w - s*q (fma), q += r*y (fma); the first leaves q within one ulp of
// w/s, so by Markstein's theorem the second gives the correctly rounded
// quotient.  That needs the residuals exact, which holds for |w| >= 2^-103;
// the caller takes FAST only when the block's amax >= 2^-84, where a smaller
// |w| has |w/s| < 2^-10 and so only its sign can reach the output (code 0 or
// 8, and a sub-block whose max is that small is clamped either way); the sign
// is restored from w.  Otherwise the IEEE divide.
template <bool FAST>
__device__ __forceinline__ int quantize_block_rows(const float4 (&v)[16], float s, uint8_t* f4s, uint8_t* e8s,
                                                   int h, int tid)
{
    const float y = 1.0f / s;
    auto quot = [&](float x) {
        if (!FAST) return x / s;
        float q = x * y;
        q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
        q = __builtin_fmaf(__builtin_fmaf(-s, q, x), y, q);
        return __builtin_copysignf(q, x);
    };
    const int c4 = tid & 31;
    const bool e8_lane = (c4 & 7) == 0;
    int nclip = 0;
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int r = i * 8 + (tid >> 5);
        const float q0 = quot(v[i].x), q1 = quot(v[i].y), q2 = quot(v[i].z), q3 = quot(v[i].w);
        const float am = max8_lanes(fmaxf(fmaxf(fabsf(q0), fabsf(q1)), fmaxf(fabsf(q2), fabsf(q3))));
        // floor(log2 am) - 2 from the exponent field; a subnormal am (field 0)
        // is far below the window
        int b = (int)((__float_as_uint(am) >> 23) & 255u) - 129;
        const bool zero = am == 0.0f;
        nclip += (!zero && b < -8 && e8_lane) ? 1 : 0;
        b = zero ? 0 : min(max(b, -8), 6);
        const float sc = __uint_as_float((uint32_t)(127 - b) << 23);   // 2^-b, exact
        *reinterpret_cast<uint16_t*>(f4s + r * kQuantPitch + h * 64 + 2 * c4) =
            (uint16_t)e2m1x4(q0 * sc, q1 * sc, q2 * sc, q3 * sc);
        if (e8_lane) e8s[r * 8 + h * 4 + (c4 >> 3)] = (uint8_t)(127 + b);
    }
    return nclip;
}

// One workgroup per 128 rows x (up to) 256 columns: two 128x128 blocks in
// turn, then 16-byte stores from LDS staging: whole 128-byte lines of codes
// per row (canonical layout), or whole 1 KiB code records and 256-byte scale
// records (packed layout, the records moe_prepack_weights would write).
__global__ __launch_bounds__(256) void k_quantize_weights(int N, int K, const float* __restrict__ w,
                                                          uint8_t* __restrict__ fp4, uint8_t* __restrict__ e8,
                                                          float* __restrict__ blk,
                                                          unsigned long long* __restrict__ clamped, int packed)
{
    __shared__ float red[2][4];
    __shared__ __align__(16) uint8_t f4s[128 * kQuantPitch];
    __shared__ __align__(16) uint8_t e8s[128 * 8];
    const int NB = N / 128, KB = K / 128, KP = (KB + 1) / 2;
    const int kp = blockIdx.x % KP;
    const int nb = (blockIdx.x / KP) % NB;
    const size_t e = blockIdx.x / ((size_t)KP * NB);
    const int nkb = min(2, KB - 2 * kp);                      // 128x128 blocks in this workgroup
    const int tid = threadIdx.x, lane = tid & 63;
    const int c4 = tid & 31;                                 // float4 column in the block row
    const size_t rowbase = e * N + (size_t)nb * 128;
    int nclip = 0;
    for (int h = 0; h < nkb; h++) {
        const int kb = 2 * kp + h;
        const float* wp = w + (rowbase + (tid >> 5)) * K + (size_t)kb * 128 + 4 * c4;
        float4 v[16];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            v[i] = *reinterpret_cast<const float4*>(wp + (size_t)i * 8 * K);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)), fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        }
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
        if (lane == 0) red[h][tid >> 6] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red[h][0], red[h][1]), fmaxf(red[h][2], red[h][3]));
        const float s = amax > 0.0f ? amax / 384.0f : 1.0f;
        if (tid == 0) blk[(e * NB + nb) * KB + kb] = s;
        nclip += amax >= 0x1p-84f ? quantize_block_rows<true>(v, s, f4s, e8s, h, tid)
                                  : quantize_block_rows<false>(v, s, f4s, e8s, h, tid);
    }
    __syncthreads();
    if (packed) {
        // code records (n-tile t of the block, chunk 2kp+h): slot sl holds row
        // 16t + sl%16, elements 32(sl/16)..+31 of the chunk
        for (int idx = tid; idx < 8 * nkb * 64; idx += 256) {
            const int t = idx / (nkb * 64), h = (idx / 64) % nkb, sl = idx % 64;
            *reinterpret_cast<uint4*>(fp4 + ((((e * (N / 16) + nb * 8 + t) * KB + 2 * kp + h) * 64) + sl) * 16) =
                *reinterpret_cast<const uint4*>(f4s + (t * 16 + (sl & 15)) * kQuantPitch + h * 64 + (sl >> 4) * 16);
        }
        // scale records (n-tile quad qd, chunk 2kp+h): byte j of lane sl's
        // dword = exponent of row (4qd+j)*16 + sl%16, sub-block sl/16
        for (int idx = tid; idx < 2 * nkb * 64; idx += 256) {
            const int qd = idx / (nkb * 64), h = (idx / 64) % nkb, sl = idx % 64;
            uint32_t d = 0;
#pragma unroll
            for (int j = 0; j < 4; j++)
                d |= (uint32_t)e8s[((qd * 4 + j) * 16 + (sl & 15)) * 8 + h * 4 + (sl >> 4)] << (8 * j);
            *reinterpret_cast<uint32_t*>(e8 + (((e * (N / 64) + nb * 2 + qd) * KB + 2 * kp + h) * 64 + sl) * 4) = d;
        }
    } else {
        // codes: 128 rows x nkb*64 bytes, 16 bytes per lane
        const int segs = nkb * 4;
        for (int idx = tid; idx < 128 * segs; idx += 256) {
            const int r = idx / segs, sg = idx % segs;
            *reinterpret_cast<uint4*>(fp4 + (rowbase + r) * (K / 2) + (size_t)kp * 128 + sg * 16) =
                *reinterpret_cast<const uint4*>(f4s + r * kQuantPitch + sg * 16);
        }
        // exponents: 4 bytes per row and block
        for (int idx = tid; idx < 128 * nkb; idx += 256) {
            const int r = idx / nkb, h = idx % nkb;
            *reinterpret_cast<uint32_t*>(e8 + (rowbase + r) * (K / 32) + (size_t)kp * 8 + h * 4) =
                *reinterpret_cast<const uint32_t*>(e8s + r * 8 + h * 4);
        }
    }
    if (nclip && clamped) atomicAdd(clamped, (unsigned long long)nclip);
}

// Test export of the weights exactly as the matrix kernels see them: one wave
// per (n-tile, chunk) record of expert `expert` runs the same block-scaled
// MFMA as the GEMM tiles against one-hot E4M3 rows (1.0 at K = 16r + row), so
// every output is a single product 1 * w * 2^b, exact in fp32; it is then
// encoded as E4M3, which is exact inside the lossless window.  out is [N][K].
__global__ __launch_bounds__(256) void k_dequant_export(int N, int K, int expert,
                                                        const uint8_t* __restrict__ fp4,
                                                        const uint8_t* __restrict__ e8,
                                                        uint8_t* __restrict__ out)
{
    const int C = K / 128;
    const int lane = threadIdx.x & 63;
    const size_t rec = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (rec >= (size_t)(N / 16) * C) return;   // whole waves
    const int c = (int)(rec % C);
    const int tile = (int)(rec / C);
    const uint4 b = *reinterpret_cast<const uint4*>(fp4 + (((size_t)expert * (N / 16) + tile) * C + c) * 1024 + lane * 16);
    const int sb = *reinterpret_cast<const int*>(e8 + (((size_t)expert * (N / 64) + tile / 4) * C + c) * 256 + lane * 4);
    const int g = lane >> 4, i = lane & 15;
    const int one = 0x38 << (8 * (i & 3));      // E4M3 1.0 in byte i%4
#pragma unroll
    for (int r = 0; r < 8; r++) {
        v8i av = {0, 0, 0, 0, 0, 0, 0, 0};
        // row i of A has its 1.0 at K = 16r + i: dwords 0-3 hold K 16g.., 4-7 hold K 64+16g..
#pragma unroll
        for (int d = 0; d < 4; d++) {
            av[d] = (r == g && (i >> 2) == d) ? one : 0;
            av[4 + d] = (r == g + 4 && (i >> 2) == d) ? one : 0;
        }
        const v4f p = mfma_e4m3_e2m1_sel(tile & 3, av, b, sb);
        // A zero product loses its sign in the accumulator (-0 + +0 = +0);
        // the E4M3 byte of a zero weight keeps the sign of its code, read from
        // the lane that holds it: lane (r/2)*16 + i, dword 2*(r%2) + g/2,
        // nibble 4*(g%2) + q.
        const int src = (r >> 1) * 16 + i;
        const uint32_t w0 = (uint32_t)__shfl((int)((r & 1) ? b.z : b.x), src);
        const uint32_t w1 = (uint32_t)__shfl((int)((r & 1) ? b.w : b.y), src);
        const uint32_t codes = (g >> 1) ? w1 : w0;
        uint32_t word = e4m3x2(p[0], p[1]) | (e4m3x2(p[2], p[3]) << 16);
#pragma unroll
        for (int q = 0; q < 4; q++) {
            const uint32_t neg = (codes >> (4 * (4 * (g & 1) + q) + 3)) & 1u;
            if (p[q] == 0.0f) word = (word & ~(0xFFu << (8 * q))) | (neg << (8 * q + 7));
        }
        *reinterpret_cast<uint32_t*>(out + (size_t)(tile * 16 + i) * K + c * 128 + 16 * r + 4 * g) = word;
    }
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
static inline unsigned blocks_for(size_t n, int per) { return (unsigned)((n + per - 1) / per); }

bool route_writes_payload(int T, int H, int E, int mode)
{
    return mode == 0 && E % 4 == 0 && H % 256 == 0 && E >= 32 && (long long)T * E <= 32768;
}

hipError_t launch_route(int T, int H, int E, int k, const uint16_t* x, const float* wr,
                        const float* bias, int mode, const int64_t* token_ids,
                        int32_t* ids, float* w, float* z, hipStream_t s, uint8_t* xq, float* xs)
{
    if (!route_writes_payload(T, H, E, mode)) xq = nullptr, xs = nullptr;
    if (mode == 1) {
        hipLaunchKernelGGL(k_route_hash, dim3(blocks_for(T, 256)), dim3(256), 0, s, T, E, k,
                           token_ids, ids, w);
        return hipGetLastError();
    }
    // Variants by the number of chains T*E (measured at H = 4096, E = 256):
    // up to 32768 (T = 128), one chain per lane (k_route_lane, 27 us; the
    // others 46 us and more); up to 131072 (T = 512), one token x one expert
    // per lane (51 us); from two blocks per CU of 128 tokens x 32 experts
    // ((T/128)*(E/32) >= 512), two tokens x eight experts per lane (W reads
    // shared by the tokens, x conversions by the experts), the block's x rows
    // staged 64 h at a time by direct-to-LDS loads (T = 8192: 324 us, against
    // 350 us with each lane reading its own x rows); from two blocks per CU of
    // 128 tokens x 16 experts, the same with four experts per lane (T = 4096 /
    // 6144: 209 / 269 us, against 239 / 357 us with one token x four experts
    // and 307 us with eight experts at 6144, which leaves CUs a block short);
    // below, one token x four experts per lane (T = 1024 / 2048: 99 / 128 us;
    // two tokens: 174 / 181 us).
    const long long chains = (long long)T * E;
    if (E % 4 != 0 || H % 256 != 0) {
        hipLaunchKernelGGL(k_route_logits_any, dim3(blocks_for((size_t)T * E, 256)), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    } else if (route_writes_payload(T, H, E, 0)) {
        constexpr int EL = 32, NTW = 2;
        const unsigned grid = (unsigned)(((T + NTW * 2 - 1) / (NTW * 2)) * ((E + EL - 1) / EL));
        hipLaunchKernelGGL((k_route_lane<EL, NTW, 256, 3>), dim3(grid), dim3(64 * (NTW + 1)), 0, s, T, H, E, x, wr,
                           bias, z, xq, xs);
    } else if (E % 32 == 0 && (size_t)((T + 127) / 128) * (E / 32) >= 512) {
        hipLaunchKernelGGL((k_route_logits<2, 8, 64, true>), dim3((T + 127) / 128, E / 32), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    } else if (E % 16 == 0 && (size_t)((T + 127) / 128) * (E / 16) >= 512) {
        hipLaunchKernelGGL((k_route_logits<2, 4, 64, true>), dim3((T + 127) / 128, E / 16), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    } else if (E % 16 == 0 && chains > 131072) {
        hipLaunchKernelGGL((k_route_logits<1, 4, 128, true>), dim3((T + 63) / 64, E / 16), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    } else if (E % 8 == 0 && chains > 131072) {
        hipLaunchKernelGGL((k_route_logits<1, 2, 256, true>), dim3((T + 63) / 64, E / 8), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    } else {
        hipLaunchKernelGGL((k_route_logits<1, 1, 256, true>), dim3((T + 63) / 64, E / 4), dim3(256), 0, s, T, H, E, x,
                           wr, bias, z);
    }
    const dim3 sg(blocks_for(T, 4));
    if (E <= 64) hipLaunchKernelGGL(k_route_select<1>, sg, dim3(256), 0, s, T, E, k, z, ids, w);
    else if (E <= 128) hipLaunchKernelGGL(k_route_select<2>, sg, dim3(256), 0, s, T, E, k, z, ids, w);
    else if (E <= 256) hipLaunchKernelGGL(k_route_select<4>, sg, dim3(256), 0, s, T, E, k, z, ids, w);
    else if (E <= 512) hipLaunchKernelGGL(k_route_select<8>, sg, dim3(256), 0, s, T, E, k, z, ids, w);
    else hipLaunchKernelGGL(k_route_select<16>, sg, dim3(256), 0, s, T, E, k, z, ids, w);
    return hipGetLastError();
}

hipError_t launch_quant_x(int T, int H, const uint16_t* x, uint8_t* xq, float* xs, hipStream_t s)
{
    hipLaunchKernelGGL(k_quant_x, dim3(blocks_for((size_t)T * H / 8, 256)), dim3(256), 0, s, T, H, x,
                       xq, xs);
    return hipGetLastError();
}

hipError_t launch_permute(int T, int k, int E, const int32_t* ids, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* hist, hipStream_t s)
{
    const int P = T * k;
    const int nblk = (P + kPermChunk - 1) / kPermChunk;
    if (nblk <= 16 && nblk * E <= 4096) {   // dynamic LDS <= 32 KiB
        const int n64 = (P + 63) / 64;
        if (n64 <= 16 && n64 * E <= 4096)
            hipLaunchKernelGGL(k_perm_small<64>, dim3(1), dim3(1024), (size_t)2 * n64 * E * 4, s, P, E, ids, offsets,
                               sorted_pair, pair_pos);
        else
            hipLaunchKernelGGL(k_perm_small<kPermChunk>, dim3(1), dim3(1024), (size_t)2 * nblk * E * 4, s, P, E, ids,
                               offsets, sorted_pair, pair_pos);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(k_perm_pass<true>, dim3(nblk), dim3(64), (size_t)E * 4, s, P, E, ids, hist,
                       sorted_pair, pair_pos);
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, s, E, nblk, hist, offsets);
    hipLaunchKernelGGL(k_perm_pass<false>, dim3(nblk), dim3(64), (size_t)E * 4, s, P, E, ids, hist,
                       sorted_pair, pair_pos);
    return hipGetLastError();
}

bool perm_tiles_one_block(int T, int k, int E)
{
    const int nblk = (T * k + kPermChunk - 1) / kPermChunk;
    return T >= 1 && nblk <= 16 && nblk * E <= 4096;
}

hipError_t launch_perm_tiles(int T, int k, int E, const int32_t* ids, int32_t* offsets, int32_t* sorted_pair,
                             int32_t* pair_pos, int MT, int NB1, int NB2, int build_queue, int lag, const FfnArgs& a,
                             int32_t* mt_expert, int32_t* mt_row0, uint32_t* queue, hipStream_t s)
{
    const int P = T * k;
    const int nblk = (P + kPermChunk - 1) / kPermChunk;
    const int n64 = (P + 63) / 64;   // 64-pair chunks when they fit the same 16 waves and LDS
    if (n64 <= 16 && n64 * E <= 4096)
        hipLaunchKernelGGL(k_perm_tiles<64>, dim3(1), dim3(1024), (size_t)2 * n64 * E * 4, s, P, E, ids, offsets,
                           sorted_pair, pair_pos, 16 * MT, NB1, NB2, build_queue, lag, mt_expert, mt_row0, a.ctrl,
                           a.done1, queue);
    else
        hipLaunchKernelGGL(k_perm_tiles<kPermChunk>, dim3(1), dim3(1024), (size_t)2 * nblk * E * 4, s, P, E, ids,
                           offsets, sorted_pair, pair_pos, 16 * MT, NB1, NB2, build_queue, lag, mt_expert, mt_row0,
                           a.ctrl, a.done1, queue);
    return hipGetLastError();
}

hipError_t launch_build_tiles(int E, int MT, int NB1, int NB2, int build_queue, int lag, const FfnArgs& a,
                              int32_t* mt_expert, int32_t* mt_row0, uint32_t* queue, hipStream_t s)
{
    hipLaunchKernelGGL(k_build_tiles, dim3(1), dim3(1024), 0, s, E, 16 * MT, NB1, NB2, build_queue, lag,
                       a.offsets, mt_expert, mt_row0, a.ctrl, a.done1, queue);
    return hipGetLastError();
}

// Kernels whose LDS exceeds the default 64 KiB limit must opt in once.
template <typename F>
static hipError_t allow_lds(F* kernel, size_t bytes, bool& done)
{
    if (done) return hipSuccess;
    hipError_t r = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    done = r == hipSuccess;
    return r;
}

template <int PHASE, int MT, int RW, int CW, bool G>
static hipError_t launch_ffn_t(const FfnArgs& a, hipStream_t s)
{
    using TL = TileLayout<MT, RW, CW>;
    static bool lds_ok = false;
    const int NB = PHASE == 1 ? a.I / (TL::HC * (G ? 1 : 2)) : a.H / TL::OC;
    const size_t lds = TL::BYTES;
    if (allow_lds(k_ffn<PHASE, MT, RW, CW, G>, lds, lds_ok) != hipSuccess) return hipErrorInvalidValue;
    // per-XCD lists: each holds at most ceil(n_mt_bound / 8) m-tiles
    const unsigned grid = a.xcd_groups ? 8u * (unsigned)NB * (unsigned)((a.n_mt_bound + 7) / 8)
                                       : (unsigned)a.n_mt_bound * NB;
    hipLaunchKernelGGL((k_ffn<PHASE, MT, RW, CW, G>), dim3(grid), dim3(TL::NT), lds, s, a, NB);
    return hipGetLastError();
}

template <int PHASE, int CW, bool G>
static hipError_t launch_ffn_cw(int MT, const FfnArgs& a, hipStream_t s)
{
    switch (MT) {
    case 1: return launch_ffn_t<PHASE, 1, 1, CW, G>(a, s);
    case 2: return launch_ffn_t<PHASE, 2, 1, CW, G>(a, s);
    case 4: return launch_ffn_t<PHASE, 4, 1, CW, G>(a, s);
    case 8: return launch_ffn_t<PHASE, 8, 2, CW, G>(a, s);
    default: return hipErrorInvalidValue;
    }
}

// Linear2 tiles do not depend on the activation: one instantiation serves both.
hipError_t launch_ffn(int phase, int MT, int CW, const FfnArgs& a, hipStream_t s)
{
    const bool g = a.act == 0;
    if (CW == 2)
        return phase == 2 ? launch_ffn_cw<2, 2, true>(MT, a, s)
                          : (g ? launch_ffn_cw<1, 2, true>(MT, a, s) : launch_ffn_cw<1, 2, false>(MT, a, s));
    if (CW == 4)
        return phase == 2 ? launch_ffn_cw<2, 4, true>(MT, a, s)
                          : (g ? launch_ffn_cw<1, 4, true>(MT, a, s) : launch_ffn_cw<1, 4, false>(MT, a, s));
    return hipErrorInvalidValue;
}

template <int MT, int RW, int CW, bool G>
static int persistent_occupancy()
{
    using TL = TileLayout<MT, RW, CW>;
    static bool lds_ok = false;
    if (allow_lds(k_ffn_persistent<MT, RW, CW, G>, TL::BYTES, lds_ok) != hipSuccess) return 1;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, k_ffn_persistent<MT, RW, CW, G>, TL::NT, TL::BYTES) !=
        hipSuccess)
        n = 1;
    return n < 1 ? 1 : n;
}

// The persistent kernel serves m-tiles of up to 64 rows (MT <= 4); 128-row
// m-tiles run as the two launches.
template <int CW, bool G>
static int persistent_occupancy_cw(int MT)
{
    switch (MT) {
    case 1: return persistent_occupancy<1, 1, CW, G>();
    case 2: return persistent_occupancy<2, 1, CW, G>();
    default: return persistent_occupancy<4, 1, CW, G>();
    }
}

int persistent_blocks_per_cu(int MT, int CW, bool gated)
{
    if (gated) return CW == 4 ? persistent_occupancy_cw<4, true>(MT) : persistent_occupancy_cw<2, true>(MT);
    return CW == 4 ? persistent_occupancy_cw<4, false>(MT) : persistent_occupancy_cw<2, false>(MT);
}

template <int MT, int RW, int CW, bool G>
static hipError_t launch_persistent_t(const FfnArgs& a, int grid, hipStream_t s)
{
    using TL = TileLayout<MT, RW, CW>;
    static bool lds_ok = false;
    if (allow_lds(k_ffn_persistent<MT, RW, CW, G>, TL::BYTES, lds_ok) != hipSuccess) return hipErrorInvalidValue;
    hipLaunchKernelGGL((k_ffn_persistent<MT, RW, CW, G>), dim3(grid), dim3(TL::NT), TL::BYTES, s, a);
    return hipGetLastError();
}

template <int CW, bool G>
static hipError_t launch_persistent_cw(int MT, const FfnArgs& a, int grid, hipStream_t s)
{
    switch (MT) {
    case 1: return launch_persistent_t<1, 1, CW, G>(a, grid, s);
    case 2: return launch_persistent_t<2, 1, CW, G>(a, grid, s);
    case 4: return launch_persistent_t<4, 1, CW, G>(a, grid, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_ffn_persistent(int MT, int CW, const FfnArgs& a, int grid, hipStream_t s)
{
    const bool g = a.act == 0;
    if (CW == 2) return g ? launch_persistent_cw<2, true>(MT, a, grid, s) : launch_persistent_cw<2, false>(MT, a, grid, s);
    if (CW == 4) return g ? launch_persistent_cw<4, true>(MT, a, grid, s) : launch_persistent_cw<4, false>(MT, a, grid, s);
    return hipErrorInvalidValue;
}

hipError_t launch_combine(int T, int H, int k, const uint16_t* y, const float* w, uint16_t* out,
                          hipStream_t s)
{
    hipLaunchKernelGGL(k_combine, dim3(blocks_for((size_t)T * H / 8, 256)), dim3(256), 0, s, T, H, k, y,
                       w, out);
    return hipGetLastError();
}

hipError_t launch_prepack(int E, int N, int K, const uint8_t* fp4_in, const uint8_t* e8_in,
                          uint8_t* fp4_out, uint8_t* e8_out, int32_t* bad, hipStream_t s)
{
    const size_t total = (size_t)E * (N / 16) * (K / 128) * 64;
    hipLaunchKernelGGL(k_prepack, dim3(blocks_for(total, 256)), dim3(256), 0, s, E, N, K, fp4_in, e8_in,
                       fp4_out, e8_out, bad);
    return hipGetLastError();
}

hipError_t launch_quantize_weights(int E, int N, int K, const float* w, uint8_t* fp4, uint8_t* e8, float* blk,
                                  unsigned long long* clamped, int packed, hipStream_t s)
{
    const size_t blocks = (size_t)E * (N / 128) * ((K / 128 + 1) / 2);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quantize_weights, dim3((unsigned)blocks), dim3(256), 0, s, N, K, w, fp4, e8, blk, clamped,
                       packed);
    return hipGetLastError();
}

hipError_t launch_dequant_export(int N, int K, int expert, const uint8_t* fp4, const uint8_t* e8,
                                 uint8_t* out, hipStream_t s)
{
    const size_t total = (size_t)(N / 16) * (K / 128) * 64;
    hipLaunchKernelGGL(k_dequant_export, dim3(blocks_for(total, 256)), dim3(256), 0, s, N, K, expert, fp4,
                       e8, out);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void k_fill_i32(int32_t* __restrict__ p, int32_t v, size_t n)
{
    const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s)
{
    hipLaunchKernelGGL(k_fill_i32, dim3(blocks_for(n, 256)), dim3(256), 0, s, p, v, n);
    return hipGetLastError();
}

int choose_mt(int T, int k, int E)
{
    // Every m-tile streams its expert's weights once, and token tiles past an
    // expert's rows are skipped, so the tile is sized to hold about 4/3 of the
    // mean rows per expert: most experts then need a single m-tile.  Measured
    // FFN times (H=4096, I=2048, E=256, top-8) put the best size there at every
    // batch from T = 128 to 8192 (T = 512: 32 rows 0.58 ms vs 16 rows 0.68;
    // T = 1024: 64 rows 0.62 vs 32 rows 0.72; T = 2048: 128 rows 0.73 vs 64 rows
    // 0.82).
    const double avg = (double)T * k / (E > 0 ? E : 1);
    if (avg <= 12.0) return 1;
    if (avg <= 24.0) return 2;
    if (avg <= 48.0) return 4;
    return 8;
}

int choose_cw(int MT, int H, int I, bool gated)
{
    // Weight-streaming small m-tiles: four wave columns whenever the shape
    // divides; one four-wave block per CU with twice the bytes per ring stage
    // measured faster than two two-wave blocks (T = 128: 0.558 -> 0.541 ms;
    // T = 512 and 1024: 5% faster).  128-row m-tiles (MFMA-bound), gated: two
    // wave columns and a two-stage ring, two blocks per CU, measured 6% faster at
    // T = 8192 than one eight-wave block with four columns and three stages,
    // though each block reads its activation rows for half the columns.  A
    // linear1 tile spans 64*CW columns of h gated, 128*CW gate-less.  (The
    // gate-less two-column linear1 tile needs more than 256 registers, so it
    // keeps the four-column layout.)
    if (MT == 8 && gated) return 2;
    return (I % (gated ? 256 : 512) == 0 && H % 512 == 0) ? 4 : 2;
}

}  // namespace v4moe
