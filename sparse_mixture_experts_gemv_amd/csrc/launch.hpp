// Host-side launchers and size plans shared by the C ABI (api.hip) and the
// kernel translation units. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace smoe {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

// ---- sparse map ----
struct SparseMapPlan {
    int L;        // routes per chunk (one workgroup of the multi-pass form)
    int nsub;     // number of chunks
    int rg;       // groups of 64 routes per wave and round (1 or 8)
    size_t ws_bytes;
};
SparseMapPlan sparse_map_plan(int64_t N, int E);
// Static per-GPU scratch of moe_sparse_map_noalloc: enough for every map with
// E <= 512 (the plan's count matrix holds at most max(2048, 2^20 / E) columns
// of E counts, plus E totals).
constexpr size_t kSparseMapNoallocScratchBytes = (size_t)4 << 20 | (size_t)4 << 10;
// Device address of this GPU's copy of that scratch (looked up once per device).
hipError_t sparse_map_noalloc_scratch(void **ptr);
hipError_t launch_sparse_map(const int32_t *ids, int N, int E, int32_t *expert_counts, int32_t *expert_offsets,
                             int32_t *sparse_rows, int32_t *slot_src, void *workspace, hipStream_t stream);

// ---- scattered FFN ----
// A block-order entry packs (M tile, N tile) as mt | nt << kOrderMtBits; an
// all-ones M field marks an empty block.
constexpr int kOrderMtBits = 20;
constexpr uint32_t kOrderMtMask = (1u << kOrderMtBits) - 1u;
constexpr int kOrderMaxNtiles = 1 << (32 - kOrderMtBits);

struct FfnPlan {
    bool atomic;               // down GEMM: fp32 atomic scatter-add (else per-route rows + combine)
    int bm_up, bm_down;        // rows per M tile of the gate+up and down GEMMs
    int bn_up, bn_down;        // columns per N tile
    int n_mtiles_up, n_mtiles_down;  // upper bounds on M tiles over all experts
    int n_ntiles_up, n_ntiles_down;
    // acc_off: fp32 [S, D] token accumulator (atomic) or fp32 [S*k, D] per-route rows
    size_t tiles_up_off, tiles_down_off, order_up_off, order_down_off, counts_off, queue_off, h_off, acc_off,
        ws_bytes;
};
FfnPlan ffn_plan(int64_t S, int64_t D, int64_t F, int64_t E, int64_t k, bool atomic);
// Whether the plan's tile counts fit the block-order entries.
inline bool ffn_plan_fits(const FfnPlan &pl) {
    return pl.n_mtiles_up < (int)kOrderMtMask && pl.n_mtiles_down < (int)kOrderMtMask &&
           pl.n_ntiles_up <= kOrderMaxNtiles && pl.n_ntiles_down <= kOrderMaxNtiles;
}
// Tile tables of up to two grouped GEMMs (tile heights bm[q]) from the
// expert offsets: per M tile (expert, row_begin, row_end), an expert-major
// block order, and the number of non-empty M tiles. A class with
// n_mtiles = 0 is skipped (its valid counter is still written).
struct TileTableArgs {
    int bm[2], n_mtiles[2], n_ntiles[2];
    int4 *tiles[2];
    uint32_t *order[2];
    int *valid[2];  // number of non-empty M tiles
    int *queue[2];  // tile claim counters of the GEMM (kQueueInts ints) to zero, or NULL
    // 0: an expert's tiles hold bm rows each and the last one the rest;
    // 1: its ceil(rows / bm) tiles share the rows evenly (sizes differ by at most one)
    int split[2];
};
// Tile claim counters of one dynamically scheduled GEMM: one per XCD, each on
// its own 64-byte line.
constexpr int kQueueStride = 16;
constexpr int kQueueInts = 8 * kQueueStride;
void launch_tile_table(const int32_t *offsets, int E, int N, const TileTableArgs &a, hipStream_t stream);
// out[t] = bf16(sum_j y[t k + j]) (fp32 rows [S*k, D] -> bf16 [S, D]), j in order
void launch_combine_rows(const float *y, uint16_t *out, int S, int D, int k, hipStream_t stream);
int pick_bm(int64_t avg);
int tiles_upper_bound(int64_t N, int64_t E, int bm);
int grid_for(size_t n, int per_block);
int device_cus();

hipError_t launch_scatter_ffn(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              int S, int D, int F, int E, int k, uint16_t *out, uint16_t *saved, void *workspace,
                              bool atomic, hipStream_t stream);

// ---- ParallelLinear ----
struct PlPlan {
    int bm, bn;                  // M tile rows, N tile columns (shared by the forward and input-gradient GEMMs)
    int n_mtiles, n_ntiles_fwd, n_ntiles_dx;
    int bm_lin, n_mtiles_lin;    // M tiles of the grouped-output forward (bm_lin >= bm, so no more tiles)
    int wg_bm, wg_bn, wg_mt, wg_nt;  // weight-gradient tiles over [D_in, D_out]
    size_t tiles_off, order_off, counts_off, rows_off, xg_off, dyg_off, ws_bytes;
};
PlPlan pl_plan(int64_t S, int64_t k, int64_t D_in, int64_t D_out, int64_t E);
inline bool pl_plan_fits(const PlPlan &pl) {
    return pl.n_mtiles < (int)kOrderMtMask && pl.n_ntiles_fwd <= kOrderMaxNtiles && pl.n_ntiles_dx <= kOrderMaxNtiles;
}
hipError_t launch_pl_fwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                         const int32_t *slot_src, int S, int k, int D_in, int D_out, int E, bool grouped_in,
                         bool grouped_out, uint16_t *y, void *workspace, hipStream_t stream);
hipError_t launch_pl_bwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                         const int32_t *slot_src, const uint16_t *dy, int S, int k, int D_in, int D_out, int E,
                         bool grouped_in, bool grouped_out, uint16_t *dx, void *dw, bool dw_bf16, float *dgates,
                         void *workspace, hipStream_t stream);

// ---- expert FFN backward ----
struct FfnBwdPlan {
    int bm_r, bm_b, bm_x, bn_b;  // tile rows of the recompute, dh and dx GEMMs; dh tile columns
    int nm_r, nm_b, nm_x;        // M tiles (upper bounds)
    int nn_r, nn_h, nn_x;        // N tiles of the recompute, dh and dx GEMMs
    int nparts;                  // router-gate partial sums per route
    size_t tiles_r, tiles_b, tiles_x, order_r, order_h, order_x, counts, ab, h, dyg, xg, rows, part, ws_bytes;
};
FfnBwdPlan ffn_bwd_plan(int64_t S, int64_t D, int64_t F, int64_t E, int64_t k);
inline bool ffn_bwd_plan_fits(const FfnBwdPlan &pl) {
    return pl.nm_r < (int)kOrderMtMask && pl.nm_b < (int)kOrderMtMask && pl.nm_x < (int)kOrderMtMask &&
           pl.nn_r <= kOrderMaxNtiles &&
           pl.nn_h <= kOrderMaxNtiles && pl.nn_x <= kOrderMaxNtiles;
}
hipError_t launch_ffn_bwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                          const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                          const uint16_t *dout, int S, int D, int F, int E, int k, uint16_t *saved, uint16_t *dx,
                          void *dw1, void *dw3, void *dw2, bool dw_bf16, float *dg, void *workspace,
                          hipStream_t stream);

// ---- router ----
size_t route_ws_bytes(int64_t S, int64_t E);
hipError_t launch_route(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, int k, int32_t *topk_ids,
                        float *topk_weights, void *workspace, hipStream_t stream);

}  // namespace smoe
