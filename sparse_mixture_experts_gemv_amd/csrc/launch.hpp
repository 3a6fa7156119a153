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
    int L;        // routes per wavefront sub-chunk
    int nsub;     // number of sub-chunks
    int nbits;    // id bits examined by match-any (covers the sentinel E)
    size_t ws_bytes;
};
SparseMapPlan sparse_map_plan(int64_t N, int E);
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
    size_t tiles_up_off, tiles_down_off, order_up_off, order_down_off, counts_off, h_off, acc_off, ws_bytes;
};
FfnPlan ffn_plan(int64_t S, int64_t D, int64_t F, int64_t E, int64_t k, bool atomic);
// Whether the plan's tile counts fit the block-order entries.
inline bool ffn_plan_fits(const FfnPlan &pl) {
    return pl.n_mtiles_up < (int)kOrderMtMask && pl.n_mtiles_down < (int)kOrderMtMask &&
           pl.n_ntiles_up <= kOrderMaxNtiles && pl.n_ntiles_down <= kOrderMaxNtiles;
}
hipError_t launch_scatter_ffn(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              int S, int D, int F, int E, int k, uint16_t *out, void *workspace, bool atomic,
                              hipStream_t stream);

// ---- router ----
size_t route_ws_bytes(int64_t S, int64_t E);
hipError_t launch_route(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, int k, int32_t *topk_ids,
                        float *topk_weights, void *workspace, hipStream_t stream);

}  // namespace smoe
