// v4moe_api.cpp -- the C ABI of libv4moe (declared in include/v4moe.h).
//
// Host side only: argument checks (plain integer and pointer tests, no
// runtime queries on the hot path; the host-launcher checks that P1 §2.1 moves
// out of Python), workspace carving, and kernel launches on the caller's
// stream.  Nothing here allocates, frees or synchronises, except the offline
// moe_prepack_weights.
//
//   P1 = "DeepSeek-V4揭秘：细粒度专家并行隐藏通信时延，FP4量化与TileLang协同优化百万Token上下文"
#include "v4moe.h"
#include "v4moe_internal.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstring>
#include <mutex>

using namespace v4moe;

namespace {

struct DeviceInfo {
    std::once_flag once;
    int ok = 0;          // 1: gfx950
    int cus = 0;
    int persist_per_cu[2][2][9] = {};   // [gated][CW == 4][MT]
    int scratch_ok = 0;  // 1: the static scratch array's address was found
};
DeviceInfo g_dev[kMaxDevices];

// One-time probe of the current device (architecture and CU count).
DeviceInfo* device_info()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    DeviceInfo* di = &g_dev[dev];
    std::call_once(di->once, [di, dev]() {
        hipDeviceProp_t prop;
        if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return;
        di->ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
        di->cus = prop.multiProcessorCount;
        for (int g = 0; g < 2; g++)
            for (int mt : {1, 2, 4})
                for (int cw : {2, 4}) di->persist_per_cu[g][cw == 4][mt] = persistent_blocks_per_cu(mt, cw, g == 1);
        di->scratch_ok = noalloc_setup_device(dev) == hipSuccess;
    });
    return di->ok ? di : nullptr;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

bool dims_ok(const v4moe_dims* d)
{
    if (!d) return false;
    if (d->T < 0 || d->T > (1 << 24)) return false;
    if (d->H < 256 || d->H > 16384 || d->H % 256) return false;
    if (d->I < 128 || d->I > 16384 || d->I % 128) return false;
    if (d->E < 1 || d->E > 1024) return false;
    if (d->topk < 1 || d->topk > 16 || d->topk > d->E) return false;
    if ((int64_t)d->T * d->topk > (1ll << 24)) return false;
    // the kernels address activations and intermediates with 32-bit offsets
    if ((int64_t)d->T * d->H >= (1ll << 31)) return false;
    if ((int64_t)d->T * d->topk * d->I >= (1ll << 31)) return false;
    if (d->act != V4MOE_ACT_SWIGLU && d->act != V4MOE_ACT_RELU2 && d->act != V4MOE_ACT_RELU) return false;
    // a gate-less linear1 tile spans at least 256 columns of h
    if (d->act != V4MOE_ACT_SWIGLU && d->I % 256) return false;
    return true;
}

// Workspace carving (offsets in bytes, each 256-aligned).
struct Layout {
    size_t z, xq, xs, sorted_pair, pair_pos, hist, mt_expert, mt_row0, ctrl, done1, queue, hq, hs, y;
    size_t total;
    int MT, CW, n_mt_bound, nblk;
};

// One 128-byte line (or more) per row of h scales, so that rows of different
// m-tiles never share a cache line.
inline int hs_stride(int I) { return ((I / 128) + 31) / 32 * 32; }

inline bool gated(const v4moe_dims* d) { return d->act == V4MOE_ACT_SWIGLU; }
// linear1 tiles per m-tile: each spans 64*CW columns of h gated, 128*CW gate-less
inline int nb1(const v4moe_dims* d, int CW) { return d->I / (64 * CW * (gated(d) ? 1 : 2)); }

Layout layout(const v4moe_dims* d)
{
    Layout L{};
    const size_t T = d->T, H = d->H, I = d->I, E = d->E, P = (size_t)d->T * d->topk;
    L.MT = choose_mt(d->T, d->topk, d->E);
    L.CW = choose_cw(L.MT, d->H, d->I, gated(d));
    const size_t M = 16 * (size_t)L.MT;
    L.n_mt_bound = (int)(P / M + (P < E ? P : E) + 1);
    L.nblk = (int)((P + kPermChunk - 1) / kPermChunk);
    const size_t NB1 = nb1(d, L.CW), NB2 = H / (128 * L.CW);
    size_t o = 0;
    auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes); return at; };
    L.z = take(T * E * 4);
    L.xq = take(T * H);
    L.xs = take(T * (H / 128) * 4);
    L.sorted_pair = take(P * 4);
    L.pair_pos = take(P * 4);
    L.hist = take((size_t)(L.nblk > 0 ? L.nblk : 1) * E * 4);
    L.mt_expert = take((size_t)L.n_mt_bound * 4);
    L.mt_row0 = take((size_t)L.n_mt_bound * 4);
    L.ctrl = take(32 * 4);
    L.done1 = take((size_t)L.n_mt_bound * 4);
    L.queue = take((size_t)L.n_mt_bound * (NB1 + NB2) * 4);
    L.hq = take(P * I);
    L.hs = take(P * hs_stride(d->I) * 4);
    L.y = take(P * H * 2);
    L.total = o;
    return L;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

bool mat_ok(const v4moe_mat& m)
{
    return m.fp4 && m.e8m0 && m.blk && aligned16(m.fp4) && aligned16(m.e8m0) && aligned16(m.blk);
}

FfnArgs ffn_args(const v4moe_dims* d, const Layout& L, uint8_t* ws, const uint8_t* xq, const float* xs,
                 const int32_t* offsets, const int32_t* sorted_pair, const v4moe_experts* w,
                 uint16_t* y)
{
    FfnArgs a{};
    a.T = d->T; a.H = d->H; a.I = d->I; a.E = d->E; a.topk = d->topk; a.act = d->act;
    a.n_mt_bound = L.n_mt_bound;
    a.xq = xq; a.xs = xs; a.offsets = offsets; a.sorted_pair = sorted_pair;
    auto mp = [](const v4moe_mat& m) {
        return MatPtr{static_cast<const uint8_t*>(m.fp4), static_cast<const uint8_t*>(m.e8m0), m.blk};
    };
    a.gate = gated(d) ? mp(w->gate) : MatPtr{};
    a.up = mp(w->up); a.down = mp(w->down);
    a.hq = ws + L.hq;
    a.hs = reinterpret_cast<float*>(ws + L.hs);
    a.hs_stride = hs_stride(d->I);
    a.y = y;
    a.mt_expert = reinterpret_cast<int32_t*>(ws + L.mt_expert);
    a.mt_row0 = reinterpret_cast<int32_t*>(ws + L.mt_row0);
    a.ctrl = reinterpret_cast<int32_t*>(ws + L.ctrl);
    a.done1 = reinterpret_cast<int32_t*>(ws + L.done1);
    a.queue = reinterpret_cast<uint32_t*>(ws + L.queue);
    return a;
}

// Backward workspace: the forward's layout, then the backward's buffers.
struct BwdLayout {
    Layout F;
    size_t ids, w, off, g, u, dys, dgu, dxs, padoff, bmt_expert, bmt_row0, bctrl, bdone1, dyT, dguT, xT, hT;
    size_t total;
    int n_mt4, ldd, gI, bm;
};

BwdLayout bwd_layout(const v4moe_dims* d)
{
    BwdLayout B{};
    B.F = layout(d);
    size_t o = B.F.total;
    auto take = [&](size_t bytes) { size_t at = o; o += up256(bytes); return at; };
    const size_t T = d->T, H = d->H, I = d->I, E = d->E, P = (size_t)d->T * d->topk;
    B.gI = d->act == V4MOE_ACT_SWIGLU ? 2 * d->I : d->I;
    B.bm = bwd_tile_rows(d->T, d->topk, d->E);
    B.n_mt4 = (int)(P / B.bm + (P < E ? P : E) + 1);    // m-tiles of the dgrad GEMMs
    B.ldd = (int)((P + 32 * E + 63) / 64 * 64);
    B.ids = take(P * 4);
    B.w = take(P * 4);
    B.off = take((E + 1) * 4);
    B.g = take(d->act == V4MOE_ACT_SWIGLU ? P * I * 4 : 0);
    B.u = take(P * I * 4);
    B.dys = take(P * H * 2);
    B.dgu = take(P * B.gI * 2);
    B.dxs = take(P * H * 4);
    B.padoff = take((E + 1) * 4);
    B.bmt_expert = take((size_t)B.n_mt4 * 4);
    B.bmt_row0 = take((size_t)B.n_mt4 * 4);
    B.bctrl = take(16 * 4);
    B.bdone1 = take((size_t)B.n_mt4 * 4);
    B.dyT = take(H * B.ldd * 2);
    B.dguT = take((size_t)B.gI * B.ldd * 2);
    B.xT = take(H * B.ldd * 2);
    B.hT = take(I * B.ldd * 2);
    (void)T;
    B.total = o;
    return B;
}

thread_local hipEvent_t t_ev_start = nullptr, t_ev_stop = nullptr;

// Outputs of the permutation when it runs fused with the tile list (small
// batches: one block for both, in place of moe_permute's launches).
struct FusedPerm {
    const int32_t* ids;
    int32_t *offsets, *sorted_pair, *pair_pos;
};

int run_ffn(const v4moe_dims* d, const Layout& L, const FfnArgs& a, uint8_t* ws, bool persistent,
            DeviceInfo* di, hipStream_t s, const FusedPerm* ff = nullptr)
{
    const int NB1 = nb1(d, L.CW), NB2 = d->H / (128 * L.CW);
    hipEvent_t ev0 = t_ev_start, ev1 = t_ev_stop;
    t_ev_start = t_ev_stop = nullptr;
    int per = di->persist_per_cu[gated(d)][L.CW == 4][L.MT];
    int grid = di->cus * (per > 0 ? per : 1);
    // Scheduling lag in waves: linear1 tiles of about six grids' worth are
    // handed out between a wave's linear1 and linear2 entries (estimate from
    // the mean number of m-tiles per expert), so linear2 tiles almost never
    // wait.  On one GPU there is no transfer for a short lag to hide: at decode
    // 1.5 grids measured 0.563 ms, 6 grids 0.557 ms, all linear1 first 0.555 ms.
    const double mt_per_expert = (double)d->T * d->topk / d->E / (16.0 * L.MT) + 0.5;
    const double items_per_wave = kWaveExperts * (mt_per_expert < 1.0 ? 1.0 : mt_per_expert) * NB1;
    const int lag = 1 + (int)(6.0 * grid / items_per_wave);
    int32_t* mt_expert = reinterpret_cast<int32_t*>(ws + L.mt_expert);
    int32_t* mt_row0 = reinterpret_cast<int32_t*>(ws + L.mt_row0);
    uint32_t* queue = reinterpret_cast<uint32_t*>(ws + L.queue);
    // Two launches with many experts: each expert's m-tiles (and every column
    // block of them) run on one XCD, so its weights and activation rows are
    // fetched into one L2 (measured 2% faster at T = 8192, E = 256).  With
    // few experts the round-robin groups would leave XCDs idle.
    FfnArgs b = a;
    b.xcd_groups = !persistent && d->E >= 64 ? 1 : 0;
    const int mode = persistent ? 1 : (b.xcd_groups ? 2 : 0);
    const hipError_t e = ff ? launch_perm_tiles(d->T, d->topk, d->E, ff->ids, ff->offsets, ff->sorted_pair,
                                                ff->pair_pos, L.MT, NB1, NB2, mode, lag, b, mt_expert, mt_row0,
                                                queue, s)
                            : launch_build_tiles(d->E, L.MT, NB1, NB2, mode, lag, b, mt_expert, mt_row0, queue, s);
    if (e != hipSuccess) return V4MOE_ELAUNCH;
    if (ev0 && hipEventRecord(ev0, s) != hipSuccess) return V4MOE_ELAUNCH;
    if (persistent) {
        const int max_items = L.n_mt_bound * (NB1 + NB2);
        if (grid > max_items) grid = max_items;
        if (launch_ffn_persistent(L.MT, L.CW, a, grid, s) != hipSuccess) return V4MOE_ELAUNCH;
    } else {
        if (launch_ffn(1, L.MT, L.CW, b, s) != hipSuccess) return V4MOE_ELAUNCH;
        if (launch_ffn(2, L.MT, L.CW, b, s) != hipSuccess) return V4MOE_ELAUNCH;
    }
    if (ev1 && hipEventRecord(ev1, s) != hipSuccess) return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

}  // namespace

namespace v4moe {

bool device_ready() { return device_info() != nullptr; }

// The layer forward on a given workspace (moe_layer_forward and
// moe_layer_forward_noalloc).
int layer_forward_ws(
    const v4moe_dims* d, const uint16_t* x, const float* w_router, const float* bias, int32_t mode,
    const int64_t* token_ids, const v4moe_experts* w, int32_t* topk_ids, float* topk_w,
    int32_t* expert_offsets, uint16_t* out, void* workspace, size_t ws_bytes, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (mode != V4MOE_ROUTE_LEARNED && mode != V4MOE_ROUTE_HASH) return V4MOE_EDIMS;
    if (!expert_offsets) return V4MOE_ENULL;
    if (d->T == 0) {
        // an empty batch: only the offsets (E+1 zeros) are written
        if (!device_info()) return V4MOE_EDEVICE;
        return launch_fill_i32(expert_offsets, 0, d->E + 1, as_stream(stream)) == hipSuccess ? V4MOE_OK
                                                                                           : V4MOE_ELAUNCH;
    }
    if (!x || !w || !topk_ids || !topk_w || !out || !workspace) return V4MOE_ENULL;
    if (mode == V4MOE_ROUTE_LEARNED && !w_router) return V4MOE_ENULL;
    if ((gated(d) && !mat_ok(w->gate)) || !mat_ok(w->up) || !mat_ok(w->down)) return V4MOE_ENULL;
    if (!aligned16(x) || !aligned16(out) || !aligned16(workspace)) return V4MOE_EALIGN;
    if (mode == V4MOE_ROUTE_LEARNED && !aligned16(w_router)) return V4MOE_EALIGN;
    const Layout L = layout(d);
    if (ws_bytes < L.total) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    hipStream_t s = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    uint8_t* xq = ws + L.xq;
    float* xs = reinterpret_cast<float*>(ws + L.xs);
    int32_t* sp = reinterpret_cast<int32_t*>(ws + L.sorted_pair);
    int32_t* pp = reinterpret_cast<int32_t*>(ws + L.pair_pos);
    uint16_t* y = reinterpret_cast<uint16_t*>(ws + L.y);
    // Small batches: the permutation and the tile list run as one block (same
    // device code, same results).  Decode-sized batches: the router also
    // writes the FP8 dispatch payload.
    const bool fuse = perm_tiles_one_block(d->T, d->topk, d->E);
    if (launch_route(d->T, d->H, d->E, d->topk, x, w_router, bias, mode, token_ids, topk_ids, topk_w,
                     reinterpret_cast<float*>(ws + L.z), s, xq, xs) != hipSuccess)
        return V4MOE_ELAUNCH;
    if (!route_writes_payload(d->T, d->H, d->E, mode) && launch_quant_x(d->T, d->H, x, xq, xs, s) != hipSuccess)
        return V4MOE_ELAUNCH;
    if (!fuse && launch_permute(d->T, d->topk, d->E, topk_ids, expert_offsets, sp, pp,
                                reinterpret_cast<int32_t*>(ws + L.hist), s) != hipSuccess)
        return V4MOE_ELAUNCH;
    const FfnArgs a = ffn_args(d, L, ws, xq, xs, expert_offsets, sp, w, y);
    const FusedPerm ff{topk_ids, expert_offsets, sp, pp};
    // The wave-scheduled persistent kernel for weight-streaming batches (m-tiles
    // of at most 64 rows); with 128-row m-tiles it measured 5-10% slower than
    // the two launches on one GPU, where there is no transfer to hide.  Both
    // run the same tiles: the results are identical.
    int rc = run_ffn(d, L, a, ws, L.MT < 8, di, s, fuse ? &ff : nullptr);
    if (rc) return rc;
    if (launch_combine(d->T, d->H, d->topk, y, topk_w, out, s) != hipSuccess) return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

}  // namespace v4moe

extern "C" {

__attribute__((visibility("default"))) size_t moe_workspace_bytes(const v4moe_dims* d)
{
    if (!dims_ok(d)) return 0;
    return layout(d).total;
}

__attribute__((visibility("default"))) void moe_time_next_ffn(void* start_event, void* stop_event)
{
    t_ev_start = static_cast<hipEvent_t>(start_event);
    t_ev_stop = static_cast<hipEvent_t>(stop_event);
}

__attribute__((visibility("default"))) const char* moe_strerror(int code)
{
    switch (code) {
    case V4MOE_OK: return "ok";
    case V4MOE_ENULL: return "a required pointer is NULL";
    case V4MOE_EDIMS: return "unsupported or inconsistent dimensions";
    case V4MOE_EALIGN: return "a pointer is not 16-byte aligned";
    case V4MOE_EWORKSPACE: return "workspace too small";
    case V4MOE_ELAUNCH: return "HIP launch or runtime call failed";
    case V4MOE_ESCALE: return "sub-block scale outside the lossless window [-8, 6]";
    case V4MOE_EDEVICE: return "current device is not gfx950";
    default: return "unknown error";
    }
}

__attribute__((visibility("default"))) int moe_route(const v4moe_dims* d, const uint16_t* x,
                                                     const float* w_router, const float* bias,
                                                     int32_t mode, const int64_t* token_ids,
                                                     int32_t* topk_ids, float* topk_w, void* workspace,
                                                     size_t ws_bytes, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (mode != V4MOE_ROUTE_LEARNED && mode != V4MOE_ROUTE_HASH) return V4MOE_EDIMS;
    if (d->T == 0) return V4MOE_OK;
    if (!topk_ids || !topk_w) return V4MOE_ENULL;
    if (mode == V4MOE_ROUTE_LEARNED && (!x || !w_router || !workspace)) return V4MOE_ENULL;
    if (mode == V4MOE_ROUTE_LEARNED && (!aligned16(x) || !aligned16(w_router) || !aligned16(workspace)))
        return V4MOE_EALIGN;
    const Layout L = layout(d);
    if (mode == V4MOE_ROUTE_LEARNED && ws_bytes < L.total) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    float* z = mode == V4MOE_ROUTE_LEARNED ? reinterpret_cast<float*>(static_cast<uint8_t*>(workspace) + L.z)
                                           : nullptr;
    if (launch_route(d->T, d->H, d->E, d->topk, x, w_router, bias, mode, token_ids, topk_ids, topk_w, z,
                     as_stream(stream)) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_permute(const v4moe_dims* d, const uint16_t* x,
                                                       const int32_t* topk_ids, int32_t* expert_offsets,
                                                       int32_t* sorted_pair, int32_t* pair_pos,
                                                       uint8_t* xq, float* xs, void* workspace,
                                                       size_t ws_bytes, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (!expert_offsets) return V4MOE_ENULL;
    if (d->T == 0) {
        // an empty batch: only the offsets (E+1 zeros) are written
        if (!device_info()) return V4MOE_EDEVICE;
        return launch_fill_i32(expert_offsets, 0, d->E + 1, as_stream(stream)) == hipSuccess ? V4MOE_OK
                                                                                           : V4MOE_ELAUNCH;
    }
    if (!x || !topk_ids || !sorted_pair || !pair_pos || !xq || !xs || !workspace) return V4MOE_ENULL;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(workspace)) return V4MOE_EALIGN;
    const Layout L = layout(d);
    if (ws_bytes < L.total) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    hipStream_t s = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    if (launch_quant_x(d->T, d->H, x, xq, xs, s) != hipSuccess) return V4MOE_ELAUNCH;
    if (launch_permute(d->T, d->topk, d->E, topk_ids, expert_offsets, sorted_pair, pair_pos,
                       reinterpret_cast<int32_t*>(ws + L.hist), s) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_expert_ffn(const v4moe_dims* d, const uint8_t* xq,
                                                          const float* xs, const int32_t* expert_offsets,
                                                          const int32_t* sorted_pair, const v4moe_experts* w,
                                                          uint16_t* y, void* workspace, size_t ws_bytes,
                                                          void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (d->T == 0) return V4MOE_OK;
    if (!xq || !xs || !expert_offsets || !sorted_pair || !w || !y || !workspace) return V4MOE_ENULL;
    if ((gated(d) && !mat_ok(w->gate)) || !mat_ok(w->up) || !mat_ok(w->down)) return V4MOE_ENULL;
    if (!aligned16(xq) || !aligned16(y) || !aligned16(workspace)) return V4MOE_EALIGN;
    const Layout L = layout(d);
    if (ws_bytes < L.total) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const FfnArgs a = ffn_args(d, L, ws, xq, xs, expert_offsets, sorted_pair, w, y);
    return run_ffn(d, L, a, ws, false, di, as_stream(stream));
}

__attribute__((visibility("default"))) int moe_combine(const v4moe_dims* d, const uint16_t* y,
                                                       const float* topk_w, uint16_t* out, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (d->T == 0) return V4MOE_OK;
    if (!y || !topk_w || !out) return V4MOE_ENULL;
    if (!aligned16(y) || !aligned16(out)) return V4MOE_EALIGN;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    if (launch_combine(d->T, d->H, d->topk, y, topk_w, out, as_stream(stream)) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_layer_forward(
    const v4moe_dims* d, const uint16_t* x, const float* w_router, const float* bias, int32_t mode,
    const int64_t* token_ids, const v4moe_experts* w, int32_t* topk_ids, float* topk_w,
    int32_t* expert_offsets, uint16_t* out, void* workspace, size_t ws_bytes, void* stream)
{
    return v4moe::layer_forward_ws(d, x, w_router, bias, mode, token_ids, w, topk_ids, topk_w, expert_offsets, out,
                                   workspace, ws_bytes, stream);
}

__attribute__((visibility("default"))) int moe_prepack_weights(const v4moe_dims* d,
                                                               const v4moe_experts* canonical,
                                                               const v4moe_experts* packed,
                                                               void* workspace, size_t ws_bytes,
                                                               void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (!canonical || !packed || !workspace) return V4MOE_ENULL;
    if ((gated(d) && (!mat_ok(canonical->gate) || !mat_ok(packed->gate))) || !mat_ok(canonical->up) ||
        !mat_ok(canonical->down) || !mat_ok(packed->up) || !mat_ok(packed->down))
        return V4MOE_ENULL;
    if (!aligned16(workspace)) return V4MOE_EALIGN;
    if (ws_bytes < 256) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    hipStream_t s = as_stream(stream);
    int32_t* bad = static_cast<int32_t*>(workspace);
    if (launch_fill_i32(bad, 0, 1, s) != hipSuccess) return V4MOE_ELAUNCH;
    const v4moe_mat* in[3] = {&canonical->gate, &canonical->up, &canonical->down};
    const v4moe_mat* out[3] = {&packed->gate, &packed->up, &packed->down};
    const int N[3] = {d->I, d->I, d->H}, K[3] = {d->H, d->H, d->I};
    for (int i = gated(d) ? 0 : 1; i < 3; i++) {
        if (launch_prepack(d->E, N[i], K[i], static_cast<const uint8_t*>(in[i]->fp4),
                           static_cast<const uint8_t*>(in[i]->e8m0),
                           static_cast<uint8_t*>(const_cast<void*>(out[i]->fp4)),
                           static_cast<uint8_t*>(const_cast<void*>(out[i]->e8m0)), bad, s) != hipSuccess)
            return V4MOE_ELAUNCH;
        if (out[i]->blk != in[i]->blk &&
            hipMemcpyAsync(const_cast<float*>(out[i]->blk), in[i]->blk,
                           (size_t)d->E * (N[i] / 128) * (K[i] / 128) * 4, hipMemcpyDeviceToDevice,
                           s) != hipSuccess)
            return V4MOE_ELAUNCH;
    }
    int32_t flag = 0;
    if (hipMemcpyAsync(&flag, bad, 4, hipMemcpyDeviceToHost, s) != hipSuccess) return V4MOE_ELAUNCH;
    if (hipStreamSynchronize(s) != hipSuccess) return V4MOE_ELAUNCH;
    return flag ? V4MOE_ESCALE : V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_quantize_weights(int32_t E, int32_t N, int32_t K,
                                                                const float* w, int32_t packed,
                                                                const v4moe_mat* out, uint64_t* clamped,
                                                                void* stream)
{
    if (!w || !out || !mat_ok(*out)) return V4MOE_ENULL;
    if (E < 1 || N < 128 || N % 128 || K < 128 || K % 128) return V4MOE_EDIMS;
    if (!aligned16(w) || !aligned16(out->fp4)) return V4MOE_EALIGN;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    if (launch_quantize_weights(E, N, K, w, static_cast<uint8_t*>(const_cast<void*>(out->fp4)),
                                static_cast<uint8_t*>(const_cast<void*>(out->e8m0)), const_cast<float*>(out->blk),
                                reinterpret_cast<unsigned long long*>(clamped), packed ? 1 : 0,
                                as_stream(stream)) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_dequant_fp8(const v4moe_mat* m, int32_t N, int32_t K,
                                                           int32_t expert, uint8_t* out, void* stream)
{
    if (!m || !out) return V4MOE_ENULL;
    if (!mat_ok(*m)) return V4MOE_ENULL;
    if (N < 64 || N % 64 || K < 128 || K % 128 || expert < 0) return V4MOE_EDIMS;
    if (!aligned16(out)) return V4MOE_EALIGN;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    if (launch_dequant_export(N, K, expert, static_cast<const uint8_t*>(m->fp4),
                              static_cast<const uint8_t*>(m->e8m0), out, as_stream(stream)) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) size_t moe_backward_workspace_bytes(const v4moe_dims* d)
{
    if (!dims_ok(d)) return 0;
    return bwd_layout(d).total;
}

__attribute__((visibility("default"))) int moe_transpose_weights(const v4moe_dims* d, const v4moe_experts* w,
                                                                 uint8_t* wt_gu, uint8_t* wt_d, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (!w || !wt_gu || !wt_d) return V4MOE_ENULL;
    if ((gated(d) && !mat_ok(w->gate)) || !mat_ok(w->up) || !mat_ok(w->down)) return V4MOE_ENULL;
    if (!aligned16(wt_gu) || !aligned16(wt_d)) return V4MOE_EALIGN;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    hipStream_t s = as_stream(stream);
    const int E = d->E, H = d->H, I = d->I, gI = gated(d) ? 2 * I : I;
    auto fp = [](const v4moe_mat& m) { return static_cast<const uint8_t*>(m.fp4); };
    auto ep = [](const v4moe_mat& m) { return static_cast<const uint8_t*>(m.e8m0); };
    if (gated(d) && launch_weights_t(E, I, H, fp(w->gate), ep(w->gate), wt_gu, gI, 0, (size_t)H * gI, s) != hipSuccess)
        return V4MOE_ELAUNCH;
    if (launch_weights_t(E, I, H, fp(w->up), ep(w->up), wt_gu, gI, gated(d) ? I : 0, (size_t)H * gI, s) != hipSuccess)
        return V4MOE_ELAUNCH;
    if (launch_weights_t(E, H, I, fp(w->down), ep(w->down), wt_d, H, 0, (size_t)I * H, s) != hipSuccess)
        return V4MOE_ELAUNCH;
    return V4MOE_OK;
}

__attribute__((visibility("default"))) int moe_layer_backward(
    const v4moe_dims* d, const uint16_t* x, const float* w_router, const float* bias, int32_t mode,
    const int64_t* token_ids, const v4moe_experts* w, const uint8_t* wt_gu, const uint8_t* wt_d,
    const uint16_t* dout, float* dx, float* dw, float* dWg, float* dWu, float* dWd, void* workspace,
    size_t ws_bytes, void* stream)
{
    if (!dims_ok(d)) return V4MOE_EDIMS;
    if (mode != V4MOE_ROUTE_LEARNED && mode != V4MOE_ROUTE_HASH) return V4MOE_EDIMS;
    if (!w || !wt_gu || !wt_d || !dWu || !dWd || !workspace || (gated(d) && !dWg)) return V4MOE_ENULL;
    if ((gated(d) && !mat_ok(w->gate)) || !mat_ok(w->up) || !mat_ok(w->down)) return V4MOE_ENULL;
    if (d->T > 0 && (!x || !dout || !dx || !dw || (mode == V4MOE_ROUTE_LEARNED && !w_router))) return V4MOE_ENULL;
    for (const void* p : {(const void*)x, (const void*)dout, (const void*)dx, (const void*)wt_gu, (const void*)wt_d,
                          (const void*)dWu, (const void*)dWd, (const void*)dWg, (const void*)workspace})
        if (p && !aligned16(p)) return V4MOE_EALIGN;
    if (mode == V4MOE_ROUTE_LEARNED && d->T > 0 && !aligned16(w_router)) return V4MOE_EALIGN;
    const BwdLayout B = bwd_layout(d);
    if (ws_bytes < B.total) return V4MOE_EWORKSPACE;
    DeviceInfo* di = device_info();
    if (!di) return V4MOE_EDEVICE;
    hipStream_t s = as_stream(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    const Layout& L = B.F;
    const int T = d->T, H = d->H, I = d->I, E = d->E, k = d->topk, gI = B.gI;
    auto at = [&](size_t off) { return ws + off; };
    int32_t* ids = reinterpret_cast<int32_t*>(at(B.ids));
    float* wts = reinterpret_cast<float*>(at(B.w));
    int32_t* offsets = reinterpret_cast<int32_t*>(at(B.off));
    uint8_t* xq = at(L.xq);
    float* xs = reinterpret_cast<float*>(at(L.xs));
    int32_t* sp = reinterpret_cast<int32_t*>(at(L.sorted_pair));
    int32_t* pp = reinterpret_cast<int32_t*>(at(L.pair_pos));
    int32_t* padoff = reinterpret_cast<int32_t*>(at(B.padoff));
    if (T > 0) {
        // the forward again, keeping what the backward needs (G, U; hq, hs; Y)
        if (launch_route(T, H, E, k, x, w_router, bias, mode, token_ids, ids, wts,
                         reinterpret_cast<float*>(at(L.z)), s) != hipSuccess)
            return V4MOE_ELAUNCH;
        if (launch_quant_x(T, H, x, xq, xs, s) != hipSuccess) return V4MOE_ELAUNCH;
        if (launch_permute(T, k, E, ids, offsets, sp, pp, reinterpret_cast<int32_t*>(at(L.hist)), s) != hipSuccess)
            return V4MOE_ELAUNCH;
        uint16_t* y = reinterpret_cast<uint16_t*>(at(L.y));
        FfnArgs a = ffn_args(d, L, ws, xq, xs, offsets, sp, w, y);
        a.g_out = gated(d) ? reinterpret_cast<float*>(at(B.g)) : nullptr;
        a.u_out = reinterpret_cast<float*>(at(B.u));
        int rc = run_ffn(d, L, a, ws, L.MT < 8, di, s);   // as in moe_layer_forward
        if (rc) return rc;
        uint16_t* dys = reinterpret_cast<uint16_t*>(at(B.dys));
        if (launch_bwd_combine(T, H, k, dout, wts, y, pp, dys, dw, s) != hipSuccess) return V4MOE_ELAUNCH;
        // m-tiles of B.bm rows over the experts' row segments
        FfnArgs b = a;
        b.ctrl = reinterpret_cast<int32_t*>(at(B.bctrl));
        b.done1 = reinterpret_cast<int32_t*>(at(B.bdone1));
        int32_t* bmte = reinterpret_cast<int32_t*>(at(B.bmt_expert));
        int32_t* bmtr = reinterpret_cast<int32_t*>(at(B.bmt_row0));
        if (launch_build_tiles(E, B.bm / 16, 1, 1, 0, 1, b, bmte, bmtr, nullptr, s) != hipSuccess)
            return V4MOE_ELAUNCH;
        BgemmArgs g{};
        g.I = I; g.H = H; g.act = d->act;
        g.mt_expert = bmte; g.mt_row0 = bmtr; g.ctrl = b.ctrl; g.offsets = offsets;
        g.g = a.g_out; g.u = a.u_out;
        uint16_t* dgu = reinterpret_cast<uint16_t*>(at(B.dgu));
        g.dgu = dgu;
        float* dxs = reinterpret_cast<float*>(at(B.dxs));
        g.dxs = dxs;
        // dh = Wd^T dY, activation derivative -> dG, dU
        g.N = I; g.K = H; g.A = dys; g.lda = H; g.Bq = wt_d; g.ldb = H; g.b_expert = (size_t)I * H;
        g.blk0 = w->down.blk;
        if (launch_bgemm(BG_DGRAD2, B.bm, g, B.n_mt4, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        // dx per row = [Wg Wu]^T [dG dU]
        g.N = H; g.K = gI; g.A = dgu; g.lda = gI; g.Bq = wt_gu; g.ldb = gI; g.b_expert = (size_t)H * gI;
        g.blk0 = gated(d) ? w->gate.blk : w->up.blk;
        g.blk1 = w->up.blk;
        if (launch_bgemm(BG_DGRAD1, B.bm, g, B.n_mt4, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        if (launch_bwd_unpermute(T, H, k, pp, dxs, dx, s) != hipSuccess) return V4MOE_ELAUNCH;
        // transposed operands of the weight gradients
        if (launch_pad_offsets(E, offsets, padoff, s) != hipSuccess) return V4MOE_ELAUNCH;
        const int P = T * k, maxc = P + 32 * E;
        uint16_t* dyT = reinterpret_cast<uint16_t*>(at(B.dyT));
        uint16_t* dguT = reinterpret_cast<uint16_t*>(at(B.dguT));
        uint16_t* xT = reinterpret_cast<uint16_t*>(at(B.xT));
        uint16_t* hT = reinterpret_cast<uint16_t*>(at(B.hT));
        if (launch_bwd_transpose(0, H, E, k, maxc, offsets, padoff, sp, dys, nullptr, nullptr, 0, dyT, B.ldd, s) !=
                hipSuccess ||
            launch_bwd_transpose(0, gI, E, k, maxc, offsets, padoff, sp, dgu, nullptr, nullptr, 0, dguT, B.ldd, s) !=
                hipSuccess ||
            launch_bwd_transpose(1, H, E, k, maxc, offsets, padoff, sp, nullptr, xq, xs, H / 128, xT, B.ldd, s) !=
                hipSuccess ||
            launch_bwd_transpose(2, I, E, k, maxc, offsets, padoff, sp, nullptr, at(L.hq),
                                 reinterpret_cast<const float*>(at(L.hs)), hs_stride(I), hT, B.ldd, s) != hipSuccess)
            return V4MOE_ELAUNCH;
        BgemmArgs wg{};
        wg.offsets = offsets; wg.padoff = padoff;
        wg.lda = wg.ldb = B.ldd;
        // weight gradients: with the same batch rule as the dgrads' tiles
        // (about 64 rows per expert or more), the kernel that holds B in registers
        wg.M = H; wg.N = I; wg.A = dyT; wg.B = hT; wg.dW = dWd;
        if (launch_bgemm(BG_WGRAD, B.bm, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        wg.M = I; wg.N = H; wg.B = xT;
        if (gated(d)) {
            wg.A = dguT; wg.dW = dWg;
            if (launch_bgemm(BG_WGRAD, B.bm, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        }
        wg.A = dguT + (gated(d) ? (size_t)I * B.ldd : 0); wg.dW = dWu;
        if (launch_bgemm(BG_WGRAD, B.bm, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
    } else {
        // no tokens: every weight gradient is zero
        if (launch_fill_i32(offsets, 0, E + 1, s) != hipSuccess) return V4MOE_ELAUNCH;
        if (launch_pad_offsets(E, offsets, padoff, s) != hipSuccess) return V4MOE_ELAUNCH;
        uint16_t* dyT = reinterpret_cast<uint16_t*>(at(B.dyT));
        BgemmArgs wg{};
        wg.offsets = offsets; wg.padoff = padoff;
        wg.lda = wg.ldb = B.ldd;
        wg.A = dyT; wg.B = dyT;
        wg.M = H; wg.N = I; wg.dW = dWd;
        if (launch_bgemm(BG_WGRAD, 64, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        wg.M = I; wg.N = H;
        if (gated(d)) {
            wg.dW = dWg;
            if (launch_bgemm(BG_WGRAD, 64, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
        }
        wg.dW = dWu;
        if (launch_bgemm(BG_WGRAD, 64, wg, 0, E, s) != hipSuccess) return V4MOE_ELAUNCH;
    }
    return V4MOE_OK;
}

}  // extern "C"
