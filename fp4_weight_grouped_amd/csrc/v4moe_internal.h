// v4moe_internal.h -- launchers shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "v4moe.h"

namespace v4moe {

// Pairs handled by one block of the permutation passes.
constexpr int kPermChunk = 256;
// Devices the library keeps per-device state for (indexed by HIP device id).
constexpr int kMaxDevices = 64;
// Bytes of the library's static per-device scratch array, the workspace of
// moe_layer_forward_noalloc (v4moe_noalloc.hip).
constexpr size_t kScratchBytes = (size_t)16 << 20;
// Experts per scheduling wave of the persistent kernel (P1 §1.2: experts are
// split into waves of a few experts each).
constexpr int kWaveExperts = 8;

struct MatPtr {
    const uint8_t* fp4;   // packed [E][N/16][K/128][64][16]
    const uint8_t* e8m0;  // packed [E][N/64][K/128][64][4]
    const float* blk;     // [E][N/128][K/128]
};

// Everything an expert-FFN tile needs.
struct FfnArgs {
    int T, H, I, E, topk;
    int act;                   // 0: SwiGLU (gate, up); 1: squared ReLU, 2: ReLU (gate-less, up only)
    int n_mt_bound;            // capacity of the m-tile list
    const uint8_t* xq;         // [T][H]   E4M3
    const float* xs;           // [T][H/128]
    const int32_t* offsets;    // [E+1]
    const int32_t* sorted_pair;// [T*topk]
    MatPtr gate, up, down;
    uint8_t* hq;               // [T*topk][I] E4M3, rows in expert-sorted order
    float* hs;                 // [T*topk][hs_stride], first I/128 used
    int hs_stride;             // floats per hs row: I/128 rounded up to a 128-byte line
    uint16_t* y;               // [T*topk][H] bf16, row = pair id
    const int32_t* mt_expert;  // [n_mt_bound] expert of each m-tile
    const int32_t* mt_row0;    // [n_mt_bound] first sorted row of each m-tile
    int32_t* ctrl;             // [0] number of m-tiles, [1] queue head, [2] queue length, [4] start of the
                               // linear2 tile list (two launches), [16+x], [24+x] XCD x's m-tile range
    int32_t* done1;            // [n_mt_bound] finished linear1 tiles per m-tile
    const uint32_t* queue;     // persistent schedule, or the per-XCD m-tile lists
    int xcd_groups;            // two-launch FFN: m-tiles grouped by XCD (k_build_tiles mode 2)
    float* g_out;              // optional [T*topk][I]: linear1 gate outputs (fp32, sorted rows), or null
    float* u_out;              // optional [T*topk][I]: linear1 up outputs, or null
};

// Routing.  With xq/xs given, the decode-sized router (route_writes_payload)
// also writes the FP8 dispatch payload of x (what launch_quant_x writes);
// otherwise they are ignored and the caller launches launch_quant_x.
bool route_writes_payload(int T, int H, int E, int mode);
hipError_t launch_route(int T, int H, int E, int k, const uint16_t* x, const float* wr,
                        const float* bias, int mode, const int64_t* token_ids,
                        int32_t* ids, float* w, float* z, hipStream_t s,
                        uint8_t* xq = nullptr, float* xs = nullptr);
hipError_t launch_quant_x(int T, int H, const uint16_t* x, uint8_t* xq, float* xs, hipStream_t s);
hipError_t launch_permute(int T, int k, int E, const int32_t* ids, int32_t* offsets,
                          int32_t* sorted_pair, int32_t* pair_pos, int32_t* hist, hipStream_t s);
hipError_t launch_build_tiles(int E, int MT, int NB1, int NB2, int build_queue, int lag,
                              const FfnArgs& a, int32_t* mt_expert, int32_t* mt_row0,
                              uint32_t* queue, hipStream_t s);
// Small batches (perm_tiles_one_block): the permutation and launch_build_tiles'
// work in one block, in place of launch_permute + launch_build_tiles.
bool perm_tiles_one_block(int T, int k, int E);
hipError_t launch_perm_tiles(int T, int k, int E, const int32_t* ids, int32_t* offsets, int32_t* sorted_pair,
                             int32_t* pair_pos, int MT, int NB1, int NB2, int build_queue, int lag, const FfnArgs& a,
                             int32_t* mt_expert, int32_t* mt_row0, uint32_t* queue, hipStream_t s);
// CW = wave columns per tile (2 or 4, from choose_cw); MT = 8 tiles also have
// two wave rows.
hipError_t launch_ffn(int phase, int MT, int CW, const FfnArgs& a, hipStream_t s);
hipError_t launch_ffn_persistent(int MT, int CW, const FfnArgs& a, int grid, hipStream_t s);
int persistent_blocks_per_cu(int MT, int CW, bool gated);
hipError_t launch_combine(int T, int H, int k, const uint16_t* y, const float* w, uint16_t* out,
                          hipStream_t s);
hipError_t launch_prepack(int E, int N, int K, const uint8_t* fp4_in, const uint8_t* e8_in,
                          uint8_t* fp4_out, uint8_t* e8_out, int32_t* bad, hipStream_t s);
hipError_t launch_quantize_weights(int E, int N, int K, const float* w, uint8_t* fp4, uint8_t* e8, float* blk,
                                  unsigned long long* clamped, int packed, hipStream_t s);
hipError_t launch_dequant_export(int N, int K, int expert, const uint8_t* fp4, const uint8_t* e8,
                                 uint8_t* out, hipStream_t s);

hipError_t launch_fill_i32(int32_t* p, int32_t v, size_t n, hipStream_t s);

// Rows per m-tile (16 * MT) used for given dimensions.
int choose_mt(int T, int k, int E);

// ---- backward (v4moe_bwd.hip) ----
enum { BG_DGRAD2 = 0, BG_DGRAD1 = 1, BG_WGRAD = 2 };
// Arguments of the grouped bf16 GEMM k_bgemm (C = sum over 128-wide K chunks
// of scale * A B^T, both operands K-contiguous).
struct BgemmArgs {
    int M, N, K;                 // WGRAD: rows, cols of dW; DGRAD: N outputs, K contraction
    int I, H, act;
    const uint16_t* A; int lda;
    const uint16_t* B; int ldb; size_t b_expert;   // B element (e, n, k) at B + e*b_expert + n*ldb + k (WGRAD)
    const uint8_t* Bq;                              // DGRAD: the same indexing, E4M3 weight bytes
    const float* blk0; const float* blk1;           // block scales (DGRAD2: down; DGRAD1: gate, up)
    const int32_t* mt_expert; const int32_t* mt_row0; const int32_t* ctrl; const int32_t* offsets;
    const int32_t* padoff;
    const float* g; const float* u;                 // forward's linear1 outputs (sorted rows, [P][I])
    uint16_t* dgu; float* dxs; float* dW;
};
hipError_t launch_bwd_combine(int T, int H, int k, const uint16_t* dout, const float* w, const uint16_t* y,
                              const int32_t* pair_pos, uint16_t* dys, float* dw, hipStream_t s);
hipError_t launch_weights_t(int E, int N, int K, const uint8_t* fp4, const uint8_t* e8, uint8_t* out, int ldo,
                            int nofs, size_t out_expert_stride, hipStream_t s);
hipError_t launch_pad_offsets(int E, const int32_t* off, int32_t* padoff, hipStream_t s);
hipError_t launch_bwd_transpose(int mode, int C, int E, int k, int max_cols, const int32_t* off,
                                const int32_t* padoff, const int32_t* sorted_pair, const uint16_t* src16,
                                const uint8_t* q8, const float* qs, int qs_stride, uint16_t* dst, int ldd,
                                hipStream_t s);
hipError_t launch_bwd_unpermute(int T, int H, int k, const int32_t* pair_pos, const float* dxs, float* dx,
                                hipStream_t s);
// DGRAD modes: grid over n_mt_bound m-tiles of bm (64 or 128) rows x N/128;
// WGRAD: bm = 128 (large batches, bwd_tile_rows) one block per expert and 128
// columns of dW with B in registers (k_wgrad), otherwise E x (M/64) x (N/128).
hipError_t launch_bgemm(int mode, int bm, const BgemmArgs& a, int n_mt_bound, int E, hipStream_t s);
// Rows per dgrad m-tile of the backward: 128 once experts average 64 rows or more.
inline int bwd_tile_rows(int T, int k, int E) { return (long long)T * k >= 64LL * E ? 128 : 64; }
// Wave columns per tile: a tile covers 64*CW columns of h in linear1 (128*CW
// gate-less) and 128*CW output columns in linear2.
int choose_cw(int MT, int H, int I, bool gated);

// ---- allocation-free layer forward (v4moe_noalloc.hip) ----
// Looks up, with device `dev` current, the address of the static scratch
// array on that device and keeps it; called once per device at set-up.
hipError_t noalloc_setup_device(int dev);
// The scratch array's device address on `dev`, or nullptr if set-up failed.
void* noalloc_scratch(int dev);
// Device set-up of the library (gfx950 check, occupancy, scratch address) for
// the current device; false if the device is unusable.
bool device_ready();
// moe_layer_forward on the given workspace (both layer-forward entry points).
int layer_forward_ws(const v4moe_dims* d, const uint16_t* x, const float* w_router, const float* bias,
                     int32_t mode, const int64_t* token_ids, const v4moe_experts* w, int32_t* topk_ids,
                     float* topk_w, int32_t* expert_offsets, uint16_t* out, void* workspace, size_t ws_bytes,
                     void* stream);

}  // namespace v4moe
