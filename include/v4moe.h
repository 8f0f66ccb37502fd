/*
 * v4moe.h -- C ABI of libv4moe: the DeepSeek-V4-style MoE layer forward on one
 * MI355X (gfx950), with FP4 (MXFP4) expert weights dequantised losslessly to
 * FP8 E4M3 for FP8 matrix-core contractions.
 *
 * Sources (cited by short tag and section):
 *   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
 *        (itsolotime.com/archives/32374)
 *   P2 = "DeepSeek V4架构学习笔记" (67808.cn/a/484462.html)
 *   P4 = "DeepSeek-V4 的暗线之二：训练一台不会失控的万亿参数机器"
 *        (blog.xieydd.top/deepseek-v4-control-part2)
 *
 * Conventions for every entry point:
 *   - All array pointers are DEVICE pointers owned by the caller; the library
 *     never allocates, frees or keeps them.  Outputs are fully overwritten.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*; NULL
 *     is the default stream) and never synchronise the host, except
 *     moe_prepack_weights, which is an offline step and synchronises.
 *   - bf16 values travel as uint16_t bit patterns; E4M3 and FP4 as bytes.
 *   - Return value: 0 on success, a negative V4MOE_E* code otherwise (no
 *     exceptions cross the ABI).  A code is returned before anything is
 *     enqueued.  Device faults surface at the caller's next synchronisation.
 *   - T = 0 is a valid no-op: only expert_offsets (E+1 zeros) is written, by
 *     moe_permute and moe_layer_forward; pointers to empty arrays may be NULL.
 *   - Results are deterministic and batch-invariant: a token's outputs do not
 *     depend on the other tokens of the batch nor on run-to-run scheduling
 *     (P1 §3.1 batch invariance, §3.2 determinism).  No atomics accumulate
 *     data; atomics only hand out work and signal readiness.
 *   - Not thread-safe per workspace: concurrent calls must use distinct
 *     workspaces.
 */
#ifndef V4MOE_H
#define V4MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Error codes. */
#define V4MOE_OK               0
#define V4MOE_ENULL           -1   /* a required pointer is NULL                       */
#define V4MOE_EDIMS           -2   /* unsupported or inconsistent dimensions            */
#define V4MOE_EALIGN          -3   /* a pointer is not 16-byte aligned                  */
#define V4MOE_EWORKSPACE      -4   /* workspace too small (see moe_workspace_bytes)     */
#define V4MOE_ELAUNCH         -5   /* a HIP launch or runtime call failed               */
#define V4MOE_ESCALE          -6   /* sub-block scale outside the lossless window       */
#define V4MOE_EDEVICE         -7   /* current device is not a gfx950                    */

/* Layer dimensions.  Requirements: 0 <= T; T*topk <= 2^24; T*H < 2^31;
 * T*topk*I < 2^31; H a multiple of 256 with 256 <= H <= 16384; I a multiple
 * of 128 with 128 <= I <= 16384; 1 <= E <= 1024; 1 <= topk <= min(E, 16). */
typedef struct {
    int32_t T;      /* tokens in the batch                          */
    int32_t H;      /* hidden size (linear1 K, linear2 N)           */
    int32_t I;      /* expert intermediate size (linear1 N, linear2 K) */
    int32_t E;      /* routed experts                               */
    int32_t topk;   /* experts per token                            */
    int32_t act;    /* expert activation, V4MOE_ACT_* (0: SwiGLU)   */
} v4moe_dims;

/* Expert activations.  SwiGLU (P1 §1.4): h = SiLU(gate x) * (up x).  The
 * gate-less ones are the cheap alternative the pages recommend (P1, the
 * hardware suggestions closing §1: an elementwise activation with no
 * exponential or division, and no gate projection so that the intermediate
 * can be wider at the same parameter count; the pages name no function):
 * h = max(up x, 0)^2 or h = max(up x, 0).  Gate-less layers have no gate
 * matrix (its pointers are ignored) and need I % 256 == 0. */
#define V4MOE_ACT_SWIGLU 0
#define V4MOE_ACT_RELU2  1
#define V4MOE_ACT_RELU   2

/* One expert weight matrix for all E experts: N output rows, K inputs.
 * P1 §4 (FP4 quantisation-aware training): FP4 E2M1 elements with a scale per
 * 1x32 sub-block, nested in 128x128 FP8 quantisation blocks.
 *
 * CANONICAL layout (what a checkpoint holds; input of moe_prepack_weights):
 *   fp4  uint8 [E][N][K/2]     K contiguous; element k in the low nibble when k is even
 *   e8m0 uint8 [E][N][K/32]    sub-block scale 2^b stored as the byte 127+b
 *   blk  fp32  [E][N/128][K/128]  scale of each 128x128 block
 * PACKED layout (output of moe_prepack_weights; what every compute entry
 * point reads).  Same byte counts; blk is unchanged.  N must be a multiple
 * of 64 (true for every matrix: N is I or H).
 *   fp4  uint8 [E][N/16][K/128][64][16]  for each expert, 16-row group n16 and
 *        128-wide K chunk c, a 1 KiB record of 64 slots of 16 bytes; slot s
 *        holds row n16*16 + s%16, elements k = c*128 + (s/16)*32 + [0, 32),
 *        in canonical nibble order (element k in byte k/2, low nibble when k
 *        is even);
 *   e8m0 uint8 [E][N/64][K/128][64][4]   for each group of four consecutive
 *        n16 and each chunk c, a 256-byte record; byte t of its dword s is the
 *        sub-block scale of slot s of n16 = 4*group + t;
 *   blk  fp32  [E][N/128][K/128]
 */
typedef struct {
    const void*  fp4;
    const void*  e8m0;
    const float* blk;
} v4moe_mat;

/* The expert weights (P1 §1.4: gate, up and down projections).
 * gate, up: N = I, K = H.  down: N = H, K = I.  gate is ignored (may be all
 * NULL) for the gate-less activations. */
typedef struct {
    v4moe_mat gate;
    v4moe_mat up;
    v4moe_mat down;
} v4moe_experts;

#define V4MOE_ROUTE_LEARNED 0
#define V4MOE_ROUTE_HASH    1

/* Workspace bytes needed by moe_route, moe_permute, moe_expert_ffn and
 * moe_layer_forward for these dimensions (host-only, pure).  Returns 0 for
 * invalid dims.  The workspace is device memory owned by the caller,
 * 16-byte aligned; its contents need no initialisation. */
size_t moe_workspace_bytes(const v4moe_dims* d);

/* Routing (P2, DeepSeekMoE notes: the affinity is sqrt(softplus(.)) in place
 * of V3's sigmoid; the early layers use hash routing).
 *   x         bf16 [T][H]
 *   w_router  fp32 [H][E]
 *   bias      fp32 [E] or NULL: added to the logits (selection and weights)
 *   mode      V4MOE_ROUTE_LEARNED: logits z[t][e] = one fp32 fused
 *             multiply-add chain over h = 0 .. H-1 ascending, starting from
 *             +0 (x exact as fp32), + bias as one fp32 add afterwards; the
 *             topk largest z are taken, ties to the lower expert id, slot j
 *             = j-th pick; a = sqrt(softplus(z)); topk_w = a / sum(a) over
 *             the picks.
 *             V4MOE_ROUTE_HASH: expert_j = splitmix64(id*topk + j) mod E,
 *             stepping +1 mod E past experts already picked; topk_w = 1/topk.
 *   token_ids int64 [T] or NULL (NULL: id = t); hash mode only.
 *   topk_ids  int32 [T][topk]   (out)
 *   topk_w    fp32  [T][topk]   (out)
 *   workspace moe_workspace_bytes(d) bytes (learned mode; may be NULL in hash mode)
 * x, w_router, workspace: 16-byte aligned. */
int moe_route(const v4moe_dims* d, const uint16_t* x, const float* w_router,
              const float* bias, int32_t mode, const int64_t* token_ids,
              int32_t* topk_ids, float* topk_w, void* workspace, size_t ws_bytes,
              void* stream);

/* Dispatch on one GPU (P1 §1.1-1.2: the FP8 dispatch stage becomes a local
 * expert-sorted permutation; P1 §1.4: FP8 dispatch payload).
 *   x              bf16 [T][H]
 *   topk_ids       int32 [T][topk] (as produced by moe_route; ids must be in [0,E))
 *   expert_offsets int32 [E+1]  (out) exclusive scan of per-expert pair counts
 *   sorted_pair    int32 [T*topk] (out) pair ids p = t*topk+j, stably sorted by expert
 *   pair_pos       int32 [T*topk] (out) inverse of sorted_pair
 *   xq             uint8 [T][H]  (out) E4M3 codes of x: per token and 128-channel
 *                  group g, s = fp32(amax/448) (1 if the group is zero) and
 *                  q = E4M3(fp32(x/s)), round to nearest even, saturating
 *   xs             fp32 [T][H/128] (out) the scales s
 * The FP8 rows are gathered by the expert FFN on load: they are never
 * materialised in expert order.  x, xq: 16-byte aligned. */
int moe_permute(const v4moe_dims* d, const uint16_t* x, const int32_t* topk_ids,
                int32_t* expert_offsets, int32_t* sorted_pair, int32_t* pair_pos,
                uint8_t* xq, float* xs, void* workspace, size_t ws_bytes, void* stream);

/* Expert FFN over all experts, unfused schedule (linear1 + SwiGLU for every
 * expert, then linear2 for every expert; P1 §1.1 stage model).
 * For each pair p routed to expert e (rows of e in sorted order):
 *   G, U = per-128-K-chunk FP8 products of xq[t] with the dequantised gate/up
 *          rows, each chunk scaled by xs[t][c] * blk[n/128][c], fp32 accumulation;
 *   h    = SiLU(G) * U  (fp32), requantised to E4M3 per 128 channels like x;
 *   y[p] = bf16 of the same chunked product of h with the down rows.
 *   y    bf16 [T*topk][H] (out), row p = t*topk + j.
 * w: PACKED weights.  xq, y and all weight arrays: 16-byte aligned. */
int moe_expert_ffn(const v4moe_dims* d, const uint8_t* xq, const float* xs,
                   const int32_t* expert_offsets, const int32_t* sorted_pair,
                   const v4moe_experts* w, uint16_t* y,
                   void* workspace, size_t ws_bytes, void* stream);

/* Combine as a weighted un-permute (P1 §1.4: BF16 combine payload; P1 §3.2:
 * no atomics):  out[t] = bf16( sum_{j=0..topk-1} topk_w[t][j] * y[t*topk+j] ),
 * summed in fp32 in increasing j.  y, out: 16-byte aligned. */
int moe_combine(const v4moe_dims* d, const uint16_t* y, const float* topk_w,
                uint16_t* out, void* stream);

/* The whole layer: route, dispatch, then the expert FFN, then the combine.
 * When experts get at most 64 rows per m-tile (weight-streaming batches) the
 * FFN is one persistent kernel that runs the experts in waves of 8 (P1 §1.2
 * and Fig. 5: the compute of wave w overlaps the gather of wave w+1 and the
 * scatter-back of finished experts); with 128-row m-tiles it is the two
 * launches of moe_expert_ffn, which measured faster there.  Same tiles and
 * arithmetic either way, so the output is bit-identical to moe_route +
 * moe_permute + moe_expert_ffn + moe_combine.
 *   topk_ids, topk_w, expert_offsets: outputs exported for checking.
 *   out bf16 [T][H]. */
int moe_layer_forward(const v4moe_dims* d, const uint16_t* x, const float* w_router,
                      const float* bias, int32_t mode, const int64_t* token_ids,
                      const v4moe_experts* w, int32_t* topk_ids, float* topk_w,
                      int32_t* expert_offsets, uint16_t* out,
                      void* workspace, size_t ws_bytes, void* stream);

/* moe_layer_forward without a caller workspace, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  Same arguments, kernels and results as
 * moe_layer_forward (bit-identical outputs); the workspace is instead a
 * static device array of the library, one per GPU, of
 * moe_noalloc_max_workspace_bytes() bytes (16 MiB: the full decode layer, H =
 * 4096, I = 2048, E = 256, top-8, fits up to T = 189), held by each GPU the
 * library runs on until the process ends.  Nothing is allocated or freed.
 * Errors: V4MOE_EDIMS for unsupported dimensions; V4MOE_EWORKSPACE when
 * moe_workspace_bytes(d) exceeds the array (nothing is enqueued); otherwise
 * as moe_layer_forward.  Every call on one GPU shares the array: calls that
 * overlap on a GPU (other streams, other host threads) race, calls on one
 * stream are ordered.  No contents need to survive between calls. */
size_t moe_noalloc_max_workspace_bytes(void);
int moe_layer_forward_noalloc(const v4moe_dims* d, const uint16_t* x, const float* w_router,
                              const float* bias, int32_t mode, const int64_t* token_ids,
                              const v4moe_experts* w, int32_t* topk_ids, float* topk_w,
                              int32_t* expert_offsets, uint16_t* out, void* stream);

/* FP32 master weights -> FP4 weights (P1 §4 and P4 §4: FP4 quantisation-aware
 * training quantises the FP32 master weights to FP4 in the forward pass;
 * element format and shared-exponent rule per the OCP MX specification the
 * pages cite).
 *   w: device fp32 [E][N][K], row-major, finite values; N % 128 == 0,
 *      K % 128 == 0; 16-byte aligned.
 *   packed: 0 writes the CANONICAL layout (fp4 [E][N][K/2], e8m0
 *      [E][N][K/32]); non-zero writes the PACKED layout the matrix kernels
 *      read, byte for byte what moe_prepack_weights makes of the canonical
 *      output (so a training step needs no separate prepack).
 *   out: device matrix in that layout plus blk [E][N/128][K/128], written in
 *      full.
 * Per 128x128 block, s = max|w| / 384 in fp32 (1 for an all-zero block), so
 * the block's largest magnitude maps to 6 * 2^6, FP4's largest value at the
 * top of the lossless window.  Per 1x32 sub-block of a row, v = w / s in fp32,
 * b = floor(log2(max|v|)) - 2, raised to -8 when below the window (such a
 * sub-block is "clamped": it keeps fewer significant codes), 0 for an
 * all-zero sub-block; each element is the E2M1 code nearest to v * 2^-b,
 * ties to the even code, saturating at 6, sign kept (-0.0 gives code 8).
 * clamped: device uint64 to which the number of clamped sub-blocks is added
 * (the caller clears it), or NULL.  Asynchronous on `stream`; allocates
 * nothing.  The output passes moe_prepack_weights' window check. */
int moe_quantize_weights(int32_t E, int32_t N, int32_t K, const float* w, int32_t packed,
                         const v4moe_mat* out, uint64_t* clamped, void* stream);

/* Offline: canonical -> packed weight layout (both device buffers of equal
 * size; blk pointers of `packed` may alias those of `canonical`).  Checks that
 * every sub-block exponent b lies in the lossless window [-8, 6] (P1 §4: the
 * FP4->FP8 conversion is exact while the sub-block scales of a block stay
 * within a bounded ratio; with E4M3 subnormals that window is b in [-8, 6]).
 * Needs a workspace of at least 256 bytes; synchronises `stream`. */
int moe_prepack_weights(const v4moe_dims* d, const v4moe_experts* canonical,
                        const v4moe_experts* packed, void* workspace, size_t ws_bytes,
                        void* stream);

/* Test export of the weights exactly as the matrix kernels consume them:
 * expert `expert` of the PACKED matrix m (N rows, K inputs; N % 64 == 0,
 * K % 128 == 0) is read through the same block-scaled FP8 x FP4 MFMA path as
 * the GEMMs and written as E4M3 bytes [N][K] in canonical row-major order
 * (P1 §4: inside the window every FP4 value times its sub-block scale is an
 * E4M3 value, so the bytes are exact; a zero keeps its code's sign). */
int moe_dequant_fp8(const v4moe_mat* m, int32_t N, int32_t K, int32_t expert,
                    uint8_t* out, void* stream);

/* ---- Backward (P1 §3 and P4 §3: the MoE backward accumulates in a fixed,
 * token-ordered sequence with no atomics; P1 §4 and P4 §4: gradients are
 * computed with the forward's FP8 weights and go straight to the FP32 master
 * weights, and the transposed weights are the same FP8 values) ---- */

/* Workspace bytes of moe_layer_backward (host-only, pure; 0 for invalid dims).
 * Device memory owned by the caller, 16-byte aligned, no initialisation. */
size_t moe_backward_workspace_bytes(const v4moe_dims* d);

/* The PACKED expert weights as transposed FP8 values, one OCP E4M3 byte each
 * (exact: inside the scale window every E2M1 code times its power-of-two
 * sub-block scale is an E4M3 value, the byte moe_dequant_fp8 gives; a zero
 * keeps its code's sign; the fp32 128x128 block scales are not applied and
 * stay in w):
 *   wt_gu: [E][H][2I] bytes with [e][h][i] = gate(e, i, h), [e][h][I + i] =
 *          up(e, i, h) (gate-less: [E][H][I] of up);
 *   wt_d:  [E][I][H] bytes with [e][i][h] = down(e, h, i).
 * Computed once per weight version and passed to moe_layer_backward (whose
 * matrix products read them as bf16, converted exactly when staged).
 * Asynchronous on `stream`; 16-byte aligned outputs. */
int moe_transpose_weights(const v4moe_dims* d, const v4moe_experts* w, uint8_t* wt_gu,
                          uint8_t* wt_d, void* stream);

/* Gradients of L = sum(dout * out) for the layer forward moe_layer_forward
 * computes on the same inputs (routing, quantisation and the FFN are
 * recomputed here).  The quantisation steps are straight-through, so
 *   dx  [T][H] fp32   = dL/dx (through the FP8 dispatch payload),
 *   dw  [T][topk] fp32 = dL/d(routing weight) = <dout_t, Y_p> (the router
 *                       itself is not differentiated),
 *   dWg, dWu [E][I][H], dWd [E][H][I] fp32 = dL/d(master weights): the
 *                       gradients with respect to the FP8 weight values
 *                       (dWg unused and may be NULL gate-less).
 * Every gradient is written in full (zeros for experts without tokens), by
 * one thread per element, in a fixed order: the result is bitwise
 * deterministic.  Products run on bf16 matrix cores with fp32 accumulation;
 * dout and the row gradients are rounded to bf16 before each product, as are
 * the forward activations (E4M3 code x scale) in the weight gradients.
 *   w: PACKED weights; wt_gu, wt_d: from moe_transpose_weights;
 *   dout: bf16 bits [T][H]; workspace: moe_backward_workspace_bytes(d).
 * Pointers 16-byte aligned. */
int moe_layer_backward(const v4moe_dims* d, const uint16_t* x, const float* w_router,
                       const float* bias, int32_t mode, const int64_t* token_ids,
                       const v4moe_experts* w, const uint8_t* wt_gu, const uint8_t* wt_d,
                       const uint16_t* dout, float* dx, float* dw, float* dWg, float* dWu,
                       float* dWd, void* workspace, size_t ws_bytes, void* stream);

/* Profiling hook (no effect on results).  start/stop are hipEvent_t handles
 * created by the caller (or NULL to clear).  The next moe_expert_ffn or
 * moe_layer_forward call made by this host thread records `start` on its
 * stream just before its expert-FFN matrix kernels (after the tile-list
 * build) and `stop` just after them, then forgets both; elapsed time between
 * them is the device time of the FFN kernels alone. */
void moe_time_next_ffn(void* start_event, void* stop_event);

/* Text for an error code. */
const char* moe_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* V4MOE_H */
