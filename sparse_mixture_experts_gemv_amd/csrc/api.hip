// C ABI entry points (declared and documented in include/moe.h): argument
// validation on the host, workspace sizing and kernel launches on the
// caller's stream. Nothing here allocates memory or synchronises the host.
#include "../../include/moe.h"
#include "launch.hpp"

namespace {

bool misaligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) != 0; }

int finish(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH; }

}  // namespace

extern "C" {

const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_INVALID_ARGUMENT: return "MOE_ERR_INVALID_ARGUMENT";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE_TOO_SMALL: return "MOE_ERR_WORKSPACE_TOO_SMALL";
        case MOE_ERR_LAUNCH: return "MOE_ERR_LAUNCH";
        case MOE_ERR_SCRATCH_LIMIT: return "MOE_ERR_SCRATCH_LIMIT";
        default: return "MOE_ERR_UNKNOWN";
    }
}

int moe_version(void) { return 100; }

size_t moe_route_workspace_bytes(int32_t S, int32_t E) {
    if (S < 0 || E < 1) return 0;
    return smoe::route_ws_bytes(S, E);
}

int moe_route_topk(const uint16_t *x, const uint16_t *w_gate, int32_t S, int32_t D, int32_t E, int32_t k,
                   int32_t *topk_ids, float *topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
    if (S < 0 || D < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (S == 0) return MOE_OK;
    if (!x || !w_gate || !topk_ids || !topk_weights || !workspace) return MOE_ERR_INVALID_ARGUMENT;
    if (misaligned(x) || misaligned(w_gate) || misaligned(topk_ids) || misaligned(topk_weights) ||
        misaligned(workspace))
        return MOE_ERR_INVALID_ARGUMENT;
    if (D % 64 != 0 || E % 8 != 0 || E > 256 || k > 16) return MOE_ERR_UNSUPPORTED;
    if ((int64_t)S * D >= ((int64_t)1 << 30) || (int64_t)S * E >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (workspace_bytes < smoe::route_ws_bytes(S, E)) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return finish(smoe::launch_route(x, w_gate, S, D, E, k, topk_ids, topk_weights, workspace,
                                     reinterpret_cast<hipStream_t>(stream)));
}

size_t moe_sparse_map_workspace_bytes(int32_t S, int32_t k, int32_t E) {
    if (S < 0 || k < 1 || E < 1) return 0;
    return smoe::align_up(smoe::sparse_map_plan((int64_t)S * k, E).ws_bytes);
}

int moe_sparse_map(const int32_t *topk_ids, int32_t S, int32_t k, int32_t E, int32_t *expert_counts,
                   int32_t *expert_offsets, int32_t *sparse_rows, int32_t *slot_src, void *workspace,
                   size_t workspace_bytes, void *stream) {
    if (S < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
    if (misaligned(expert_counts) || misaligned(expert_offsets)) return MOE_ERR_INVALID_ARGUMENT;
    if (E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    if (N >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    if (N > 0) {
        if (!topk_ids || !sparse_rows || !slot_src || !workspace) return MOE_ERR_INVALID_ARGUMENT;
        if (misaligned(topk_ids) || misaligned(sparse_rows) || misaligned(slot_src) || misaligned(workspace))
            return MOE_ERR_INVALID_ARGUMENT;
        if (workspace_bytes < smoe::sparse_map_plan(N, E).ws_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    }
    return finish(smoe::launch_sparse_map(topk_ids, (int)N, E, expert_counts, expert_offsets, sparse_rows, slot_src,
                                          workspace, reinterpret_cast<hipStream_t>(stream)));
}

int moe_sparse_map_noalloc(const int32_t *topk_ids, int32_t S, int32_t k, int32_t E, int32_t *expert_counts,
                           int32_t *expert_offsets, int32_t *sparse_rows, int32_t *slot_src, void *stream) {
    if (S < 0 || k < 1 || E < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (!expert_counts || !expert_offsets) return MOE_ERR_INVALID_ARGUMENT;
    if (misaligned(expert_counts) || misaligned(expert_offsets)) return MOE_ERR_INVALID_ARGUMENT;
    if (E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    if (N >= ((int64_t)1 << 31)) return MOE_ERR_UNSUPPORTED;
    void *scratch = nullptr;
    if (N > 0) {
        if (!topk_ids || !sparse_rows || !slot_src) return MOE_ERR_INVALID_ARGUMENT;
        if (misaligned(topk_ids) || misaligned(sparse_rows) || misaligned(slot_src)) return MOE_ERR_INVALID_ARGUMENT;
        if (smoe::sparse_map_plan(N, E).ws_bytes > smoe::kSparseMapNoallocScratchBytes) return MOE_ERR_SCRATCH_LIMIT;
        // this GPU's copy of the library's static scratch (no allocation; looked up once per device)
        if (smoe::sparse_map_noalloc_scratch(&scratch) != hipSuccess) return MOE_ERR_LAUNCH;
    }
    // the kernels write every count they later read: the scratch needs no clearing
    return finish(smoe::launch_sparse_map(topk_ids, (int)N, E, expert_counts, expert_offsets, sparse_rows, slot_src,
                                          scratch, reinterpret_cast<hipStream_t>(stream)));
}

size_t moe_scatter_ffn_workspace_bytes(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1) return 0;
    return smoe::ffn_plan(S, D, F, E, k, false).ws_bytes;
}

size_t moe_scatter_ffn_workspace_bytes_atomic(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1) return 0;
    return smoe::ffn_plan(S, D, F, E, k, true).ws_bytes;
}

int moe_scatter_ffn_fwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                        const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                        int32_t S, int32_t D, int32_t F, int32_t E, int32_t k, uint16_t *out, void *workspace,
                        size_t workspace_bytes, void *stream) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (S == 0) return MOE_OK;
    if (!x || !w1 || !w3 || !w2 || !topk_weights || !expert_offsets || !slot_src || !out || !workspace)
        return MOE_ERR_INVALID_ARGUMENT;
    if (misaligned(x) || misaligned(w1) || misaligned(w3) || misaligned(w2) || misaligned(topk_weights) ||
        misaligned(expert_offsets) || misaligned(slot_src) || misaligned(out) || misaligned(workspace))
        return MOE_ERR_INVALID_ARGUMENT;
    if (D % 64 != 0 || F % 64 != 0 || E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    // 32-bit buffer offsets: x, each expert matrix and each tile's rows of h stay below 2 GiB
    if (N >= ((int64_t)1 << 31) || (int64_t)S * D >= ((int64_t)1 << 30) || (int64_t)D * F >= ((int64_t)1 << 30))
        return MOE_ERR_UNSUPPORTED;
    // the per-route-rows path when the workspace holds its fp32 [S*k, D]
    // rows, else the atomic scatter-add path
    const smoe::FfnPlan rows = smoe::ffn_plan(S, D, F, E, k, false);
    const smoe::FfnPlan atomic = smoe::ffn_plan(S, D, F, E, k, true);
    if (!smoe::ffn_plan_fits(rows)) return MOE_ERR_UNSUPPORTED;
    bool use_atomic;
    if (workspace_bytes >= rows.ws_bytes) use_atomic = false;
    else if (workspace_bytes >= atomic.ws_bytes) use_atomic = true;
    else return MOE_ERR_WORKSPACE_TOO_SMALL;
    return finish(smoe::launch_scatter_ffn(x, w1, w3, w2, topk_weights, expert_offsets, slot_src, S, D, F, E, k, out,
                                           nullptr, workspace, use_atomic, reinterpret_cast<hipStream_t>(stream)));
}

int moe_scatter_ffn_fwd_train(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              int32_t S, int32_t D, int32_t F, int32_t E, int32_t k, uint16_t *out,
                              uint16_t *saved_activations, void *workspace, size_t workspace_bytes, void *stream) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (S == 0) return MOE_OK;
    if (!x || !w1 || !w3 || !w2 || !topk_weights || !expert_offsets || !slot_src || !out || !workspace ||
        !saved_activations)
        return MOE_ERR_INVALID_ARGUMENT;
    if (misaligned(x) || misaligned(w1) || misaligned(w3) || misaligned(w2) || misaligned(topk_weights) ||
        misaligned(expert_offsets) || misaligned(slot_src) || misaligned(out) || misaligned(workspace) ||
        misaligned(saved_activations))
        return MOE_ERR_INVALID_ARGUMENT;
    if (D % 64 != 0 || F % 64 != 0 || E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    // as the forward, and the saved a | b rows (2F per slot) below 2 GiB
    if (N >= ((int64_t)1 << 31) || (int64_t)S * D >= ((int64_t)1 << 30) || (int64_t)D * F >= ((int64_t)1 << 30) ||
        N * 2 * F >= ((int64_t)1 << 30))
        return MOE_ERR_UNSUPPORTED;
    const smoe::FfnPlan rows = smoe::ffn_plan(S, D, F, E, k, false);
    if (!smoe::ffn_plan_fits(rows)) return MOE_ERR_UNSUPPORTED;
    if (workspace_bytes < rows.ws_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return finish(smoe::launch_scatter_ffn(x, w1, w3, w2, topk_weights, expert_offsets, slot_src, S, D, F, E, k, out,
                                           saved_activations, workspace, false, reinterpret_cast<hipStream_t>(stream)));
}

size_t moe_scatter_ffn_bwd_workspace_bytes(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1) return 0;
    return smoe::ffn_bwd_plan(S, D, F, E, k).ws_bytes;
}

namespace {

int ffn_bwd_impl(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                 const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                 const uint16_t *dout, int32_t S, int32_t D, int32_t F, int32_t E, int32_t k,
                 uint16_t *saved_activations, uint16_t *dx, void *dw1, void *dw3, void *dw2, bool dw_bf16,
                 float *d_topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
    if (S < 0 || D < 1 || F < 1 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARGUMENT;
    if (!dx && !dw1 && !dw3 && !dw2 && !d_topk_weights) return MOE_ERR_INVALID_ARGUMENT;
    if (!w1 || !w3 || !w2 || !expert_offsets || !workspace) return MOE_ERR_INVALID_ARGUMENT;
    if (S > 0 && (!x || !topk_weights || !slot_src || !dout)) return MOE_ERR_INVALID_ARGUMENT;
    const void *ptrs[] = {x, w1, w3, w2, topk_weights, expert_offsets, slot_src, dout, dx, dw1, dw3, dw2,
                          d_topk_weights, workspace, saved_activations};
    for (const void *q : ptrs)
        if (q && misaligned(q)) return MOE_ERR_INVALID_ARGUMENT;
    if (D % 64 != 0 || F % 64 != 0 || E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    // 32-bit buffer offsets: every row buffer and each expert matrix stay below 2 GiB
    if (N * (int64_t)(D > 2 * F ? D : 2 * F) >= ((int64_t)1 << 30) || (int64_t)S * D >= ((int64_t)1 << 30) ||
        (int64_t)D * F >= ((int64_t)1 << 30))
        return MOE_ERR_UNSUPPORTED;
    const smoe::FfnBwdPlan pl = smoe::ffn_bwd_plan(S, D, F, E, k);
    if (!smoe::ffn_bwd_plan_fits(pl)) return MOE_ERR_UNSUPPORTED;
    if (workspace_bytes < pl.ws_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    if (S == 0 && !dw1 && !dw3 && !dw2) return MOE_OK;  // with a weight gradient requested, zeros are written
    return finish(smoe::launch_ffn_bwd(x, w1, w3, w2, topk_weights, expert_offsets, slot_src, dout, S, D, F, E, k,
                                       saved_activations, dx, dw1, dw3, dw2, dw_bf16, d_topk_weights, workspace,
                                       reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int moe_scatter_ffn_bwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                        const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                        const uint16_t *dout, int32_t S, int32_t D, int32_t F, int32_t E, int32_t k,
                        uint16_t *saved_activations, uint16_t *dx, float *dw1, float *dw3, float *dw2,
                        float *d_topk_weights, void *workspace, size_t workspace_bytes, void *stream) {
    return ffn_bwd_impl(x, w1, w3, w2, topk_weights, expert_offsets, slot_src, dout, S, D, F, E, k,
                        saved_activations, dx, dw1, dw3, dw2, false, d_topk_weights, workspace, workspace_bytes,
                        stream);
}

int moe_scatter_ffn_bwd_bf16w(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              const uint16_t *dout, int32_t S, int32_t D, int32_t F, int32_t E, int32_t k,
                              uint16_t *saved_activations, uint16_t *dx, uint16_t *dw1, uint16_t *dw3,
                              uint16_t *dw2, float *d_topk_weights, void *workspace, size_t workspace_bytes,
                              void *stream) {
    return ffn_bwd_impl(x, w1, w3, w2, topk_weights, expert_offsets, slot_src, dout, S, D, F, E, k,
                        saved_activations, dx, dw1, dw3, dw2, true, d_topk_weights, workspace, workspace_bytes,
                        stream);
}

size_t moe_parallel_linear_workspace_bytes(int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E) {
    if (S < 0 || k < 1 || D_in < 1 || D_out < 1 || E < 1) return 0;
    return smoe::pl_plan(S, k, D_in, D_out, E).ws_bytes;
}

namespace {

// Shared checks of the ParallelLinear calls; returns MOE_OK or an error.
int pl_check(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
             const int32_t *slot_src, int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E,
             int32_t grouped_in, int32_t grouped_out, void *workspace, size_t workspace_bytes) {
    if (S < 0 || k < 1 || E < 1 || k > E || D_in < 1 || D_out < 1) return MOE_ERR_INVALID_ARGUMENT;
    if ((grouped_in != 0 && grouped_in != 1) || (grouped_out != 0 && grouped_out != 1))
        return MOE_ERR_INVALID_ARGUMENT;
    if (!w || !expert_offsets || !workspace || (S > 0 && (!x || !slot_src))) return MOE_ERR_INVALID_ARGUMENT;
    if ((x && misaligned(x)) || misaligned(w) || misaligned(expert_offsets) || (slot_src && misaligned(slot_src)) ||
        misaligned(workspace) || (gates && misaligned(gates)))
        return MOE_ERR_INVALID_ARGUMENT;
    if (D_in % 64 != 0 || D_out % 64 != 0 || E > 1024) return MOE_ERR_UNSUPPORTED;
    const int64_t N = (int64_t)S * k;
    // 32-bit buffer offsets: every row buffer and each expert matrix stay below 2 GiB
    if (N * (int64_t)(D_in > D_out ? D_in : D_out) >= ((int64_t)1 << 30) ||
        (int64_t)D_in * D_out >= ((int64_t)1 << 30))
        return MOE_ERR_UNSUPPORTED;
    const smoe::PlPlan pl = smoe::pl_plan(S, k, D_in, D_out, E);
    if (!smoe::pl_plan_fits(pl)) return MOE_ERR_UNSUPPORTED;
    if (workspace_bytes < pl.ws_bytes) return MOE_ERR_WORKSPACE_TOO_SMALL;
    return MOE_OK;
}

}  // namespace

int moe_parallel_linear_fwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                            const int32_t *slot_src, int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E,
                            int32_t grouped_in, int32_t grouped_out, uint16_t *y, void *workspace,
                            size_t workspace_bytes, void *stream) {
    if (S < 0 || k < 1 || E < 1 || k > E || D_in < 1 || D_out < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (S == 0) return MOE_OK;
    if (!y || misaligned(y)) return MOE_ERR_INVALID_ARGUMENT;
    const int st = pl_check(x, w, gates, expert_offsets, slot_src, S, k, D_in, D_out, E, grouped_in, grouped_out,
                            workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    return finish(smoe::launch_pl_fwd(x, w, gates, expert_offsets, slot_src, S, k, D_in, D_out, E, grouped_in != 0,
                                      grouped_out != 0, y, workspace, reinterpret_cast<hipStream_t>(stream)));
}

namespace {

int pl_bwd_impl(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                const int32_t *slot_src, const uint16_t *dy, int32_t S, int32_t k, int32_t D_in, int32_t D_out,
                int32_t E, int32_t grouped_in, int32_t grouped_out, uint16_t *dx, void *dw, bool dw_bf16,
                float *dgates, void *workspace, size_t workspace_bytes, void *stream) {
    if (S < 0 || k < 1 || E < 1 || k > E || D_in < 1 || D_out < 1) return MOE_ERR_INVALID_ARGUMENT;
    if (!dx && !dw && !dgates) return MOE_ERR_INVALID_ARGUMENT;
    if (S == 0 && !dw) return MOE_OK;  // with dw, the zero gradient is still written
    if ((S > 0 && !dy) || (dy && misaligned(dy)) || (dx && misaligned(dx)) || (dw && misaligned(dw)) ||
        (dgates && misaligned(dgates)))
        return MOE_ERR_INVALID_ARGUMENT;
    const int st = pl_check(x, w, gates, expert_offsets, slot_src, S, k, D_in, D_out, E, grouped_in, grouped_out,
                            workspace, workspace_bytes);
    if (st != MOE_OK) return st;
    return finish(smoe::launch_pl_bwd(x, w, gates, expert_offsets, slot_src, dy, S, k, D_in, D_out, E,
                                      grouped_in != 0, grouped_out != 0, dx, dw, dw_bf16, dgates, workspace,
                                      reinterpret_cast<hipStream_t>(stream)));
}

}  // namespace

int moe_parallel_linear_bwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                            const int32_t *slot_src, const uint16_t *dy, int32_t S, int32_t k, int32_t D_in,
                            int32_t D_out, int32_t E, int32_t grouped_in, int32_t grouped_out, uint16_t *dx,
                            float *dw, float *dgates, void *workspace, size_t workspace_bytes, void *stream) {
    return pl_bwd_impl(x, w, gates, expert_offsets, slot_src, dy, S, k, D_in, D_out, E, grouped_in, grouped_out, dx,
                       dw, false, dgates, workspace, workspace_bytes, stream);
}

int moe_parallel_linear_bwd_bf16w(const uint16_t *x, const uint16_t *w, const float *gates,
                                  const int32_t *expert_offsets, const int32_t *slot_src, const uint16_t *dy,
                                  int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E, int32_t grouped_in,
                                  int32_t grouped_out, uint16_t *dx, uint16_t *dw, float *dgates, void *workspace,
                                  size_t workspace_bytes, void *stream) {
    return pl_bwd_impl(x, w, gates, expert_offsets, slot_src, dy, S, k, D_in, D_out, E, grouped_in, grouped_out, dx,
                       dw, true, dgates, workspace, workspace_bytes, stream);
}

}  // extern "C"
