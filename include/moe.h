/*
 * moe.h -- C ABI of the dropless sparse Mixture-of-Experts forward path for
 * AMD Instinct MI355X (gfx950).
 *
 * The forward pass has four stages. This library exports them as three calls
 * (plus, below, the FFN's backward and the general ParallelLinear primitive
 * with its backward):
 *
 *   moe_route_topk       router: H(X) = Softmax(TopK(X W_gate, k))
 *                        (ScatterMoE Guide, section "1. The Dynamic Routing
 *                        Imbalance Dilemma", equation H(X)).
 *   moe_sparse_map       per-expert histogram, exclusive scan and stable
 *                        route -> slot assignment (same page, section
 *                        "2. Grouped Coordinate Indexing Without Padding",
 *                        equations Histogram(e) and Offsets(e); Fast-LLM pull
 *                        request "Add scalable sparse map kernel", sections
 *                        "Solution" and "Usage": the (expert_ends,
 *                        expert_pad_begins, sparse_rows) triple).
 *   moe_scatter_ffn_fwd  SwiGLU experts over gathered token rows with no
 *                        [S*k, D] copy and no padding, then the
 *                        router-weighted scatter-add back to token order
 *                        (ScatterMoE Guide, figure "The ParallelLinear Core
 *                        Abstraction" and section "1. The Anatomy of
 *                        ParallelLinear": ParallelLinear(X, W, I, G); section
 *                        "2. The Hidden Cost of Activation Materialization").
 *
 * Notation: S tokens, D model width, F expert FFN width, E experts, k experts
 * per token. f = s*k + j is the flat route index of token s's j-th expert. A
 * "slot" is a row of the expert-sorted order: slots [offsets[e], offsets[e+1])
 * belong to expert e and are ordered by f (a stable sort).
 *
 * Conventions for every call:
 *  - All array pointers are DEVICE pointers (hipMalloc'd or torch CUDA
 *    tensors), row-major, 16-byte aligned. bf16 values are passed as their
 *    raw 16-bit patterns (uint16_t).
 *  - `stream` is a hipStream_t (NULL = the default stream). Every call only
 *    enqueues kernels on it (no memset or copy nodes: every clear is a
 *    kernel), never synchronises the host and never allocates, so a sequence
 *    of calls may be recorded into a HIP graph by stream capture and
 *    replayed; a replay reads and writes the same buffers.
 *  - The caller owns every buffer. Inputs are read only; outputs are fully
 *    overwritten. `workspace` is caller-allocated scratch whose contents are
 *    undefined before and after a call; calls in flight at the same time
 *    must use different workspaces.
 *  - Errors: argument checks happen on the host before anything is
 *    enqueued: NULL pointer, misaligned pointer, S < 0, E < 1, k < 1, k > E
 *    -> MOE_ERR_INVALID_ARGUMENT; shapes outside the kernels' limits ->
 *    MOE_ERR_UNSUPPORTED; workspace too small -> MOE_ERR_WORKSPACE_TOO_SMALL;
 *    a failed launch -> MOE_ERR_LAUNCH. S == 0 enqueues nothing (or, for the
 *    sparse map, only the zeroing of counts and offsets) and returns MOE_OK.
 *  - Device-side preconditions are NOT checked on the GPU: expert ids lie in
 *    [0, E) and are distinct within a token; the map passed to
 *    moe_scatter_ffn_fwd was built from the same ids; S*k < 2^31.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_LAUNCH = 4,
    MOE_ERR_SCRATCH_LIMIT = 5 /* a no-allocation call needs more than its static scratch holds */
} moe_status;

/* Human-readable name of a status code (static string, never NULL). */
const char *moe_status_str(int status);

/* Library version as major*10000 + minor*100 + patch. */
int moe_version(void);

/*
 * Workspace bytes moe_route_topk needs for these sizes (partial router
 * logits in fp32, [splits, S, E], for E > 16; zero for E <= 16). Pure host
 * function.
 */
size_t moe_route_workspace_bytes(int32_t S, int32_t E);

/*
 * Router (ScatterMoE Guide, section "1. The Dynamic Routing Imbalance
 * Dilemma", equation H(X); the page's FFN block computes the same thing as
 * softmax, top-k, renormalise).
 *   logits[s, e] = sum_d x[s, d] * w_gate[d, e]      (bf16 in, fp32 sum;
 *                  the order of the fp32 sum is fixed, so ids are
 *                  reproducible run to run)
 *   topk_ids[s, 0..k-1]  = the k largest logits, descending; equal logits
 *                          rank the lower expert id first
 *   topk_weights[s, j]   = exp(l_j - l_0) / sum_j' exp(l_j' - l_0)  (fp32)
 * x [S, D] bf16; w_gate [D, E] bf16; topk_ids [S, k] int32;
 * topk_weights [S, k] fp32; workspace >= moe_route_workspace_bytes(S, E).
 * Limits: D % 64 == 0, E % 8 == 0, E <= 256, k <= 16, S*D < 2^30
 * (else UNSUPPORTED).
 */
int moe_route_topk(const uint16_t *x, const uint16_t *w_gate, int32_t S, int32_t D, int32_t E, int32_t k,
                   int32_t *topk_ids, float *topk_weights, void *workspace, size_t workspace_bytes,
                   void *stream);

/* Workspace bytes moe_sparse_map needs. Pure host function. */
size_t moe_sparse_map_workspace_bytes(int32_t S, int32_t k, int32_t E);

/*
 * Sparse map (ScatterMoE Guide, section "2. Grouped Coordinate Indexing
 * Without Padding"; Fast-LLM scalable sparse map):
 *   expert_counts[e]   = Histogram(e) = #{f : topk_ids[f] == e}
 *   expert_offsets[e]  = Offsets(e) = sum_{e' < e} expert_counts[e'];
 *                        expert_offsets[E] = S*k. Fast-LLM's expert_ends are
 *                        expert_offsets[1..E]; expert_pad_begins equal the
 *                        ends (dropless: no padding).
 *   sparse_rows[f]     = slot of route f = expert_offsets[e] +
 *                        #{f' < f : topk_ids[f'] == e}, e = topk_ids[f]
 *   slot_src[slot]     = f (inverse permutation of sparse_rows)
 * The assignment is deterministic and stable (flat route order), so the
 * result is bit-identical from run to run.
 * topk_ids [S, k] int32 in [0, E); expert_counts [E]; expert_offsets [E+1];
 * sparse_rows, slot_src [S*k] (all int32).
 * Limits: E <= 1024 (else UNSUPPORTED).
 */
int moe_sparse_map(const int32_t *topk_ids, int32_t S, int32_t k, int32_t E, int32_t *expert_counts,
                   int32_t *expert_offsets, int32_t *sparse_rows, int32_t *slot_src, void *workspace,
                   size_t workspace_bytes, void *stream);

/*
 * moe_sparse_map without a workspace argument, for callers that cannot
 * allocate device memory (code being captured into a HIP graph, serving loops
 * that forbid hipMalloc, harnesses without an allocator). It runs the same
 * kernels and gives the same outputs, bit for bit, as moe_sparse_map; the
 * per-chunk count matrix that moe_sparse_map keeps in its workspace lives here
 * in a static device array of the library instead: 4 MiB + 4 KiB per GPU,
 * reserved in each GPU's memory when the library's code is loaded there and
 * held until the process ends. The call itself allocates nothing.
 *  - That scratch serves exactly the maps whose
 *    moe_sparse_map_workspace_bytes() is at most its size: every map with
 *    E <= 512, every map of fewer than 2^20 routes, and at E = 1024 maps of
 *    up to 2^22 routes. A map that needs more returns MOE_ERR_SCRATCH_LIMIT
 *    before anything is enqueued (moe_sparse_map with a workspace of
 *    moe_sparse_map_workspace_bytes() serves those).
 *  - Every call on one GPU uses that GPU's single copy of the scratch, and the
 *    kernels write every count they read, so no clearing is needed between
 *    calls. Calls that overlap in time on one GPU (for example on two
 *    streams) race on the scratch and give undefined results: serialise them.
 *  - The first call on a device looks up the scratch's device address (with
 *    that device current); a failure there returns MOE_ERR_LAUNCH.
 * Arguments, outputs, limits and the other errors as moe_sparse_map.
 */
int moe_sparse_map_noalloc(const int32_t *topk_ids, int32_t S, int32_t k, int32_t E, int32_t *expert_counts,
                           int32_t *expert_offsets, int32_t *sparse_rows, int32_t *slot_src, void *stream);

/*
 * Workspace bytes for the default combine of moe_scatter_ffn_fwd: the
 * intermediate h [S*k, F] bf16 in slot order, the router-weighted down
 * projection of every route y [S*k, D] fp32, a tile table and the gate+up
 * GEMM's tile-claim counters (rewritten by every call). The input
 * token rows are never replicated (x is read in place by index). Pure host
 * function.
 */
size_t moe_scatter_ffn_workspace_bytes(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k);

/*
 * Smaller workspace that selects the atomic scatter-add combine: h, an fp32
 * token accumulator [S, D] and a tile table. No term is proportional to
 * S*k*D. Pure host function.
 */
size_t moe_scatter_ffn_workspace_bytes_atomic(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k);

/*
 * Scattered SwiGLU experts with weighted scatter-add combine (ScatterMoE
 * Guide, "The ParallelLinear Core Abstraction": gather rows of X by index,
 * tile GEMM against W[e], scale by the router coefficient, accumulate into
 * the token's output row; section "2. The Hidden Cost of Activation
 * Materialization": SwiGLU experts).
 * For every slot r of expert e (offsets[e] <= r < offsets[e+1]), with
 * f = slot_src[r] and token t = f / k:
 *   h[r, :]  = bf16( SiLU(x[t, :] W1[e]) * (x[t, :] W3[e]) )   (fp32 sums)
 *   y_f      = topk_weights[f] * (h[r, :] W2[e])                 (fp32)
 *   out[t,:] = bf16( sum over the k routes f of token t of y_f )  (rounded once)
 * The combine runs one of two ways, chosen by workspace_bytes:
 *  - workspace_bytes >= moe_scatter_ffn_workspace_bytes(): the down
 *    projection stores y_f to row f of an fp32 [S*k, D] buffer and a combine
 *    pass adds the k rows of each token in the order j = 0 .. k-1. The
 *    output is bitwise reproducible from run to run.
 *  - else, workspace_bytes >= moe_scatter_ffn_workspace_bytes_atomic(): the
 *    down projection adds y_f into an fp32 [S, D] token accumulator with
 *    atomics (the in-place scatter-add of the ScatterMoE kernel); the order
 *    of the k additions is not fixed, so the last fp32 bit may vary.
 * x [S, D] bf16; w1, w3 [E, D, F] bf16; w2 [E, F, D] bf16 (each expert's
 * matrix is [D_in, D_out] with D_out contiguous); topk_weights [S, k] fp32;
 * expert_offsets [E+1] and slot_src [S*k] from moe_sparse_map on the same
 * ids; out [S, D] bf16 (fully written).
 * The gate+up tiles are handed out at run time from per-XCD queues whose
 * counters live in the workspace, so two calls in flight at once (on
 * different streams) need different workspaces, as for h and y.
 * Limits: D % 64 == 0, F % 64 == 0, E <= 1024, S*D < 2^30, D*F < 2^30
 * (32-bit buffer offsets), D <= 2^19, F <= 2^19 and fewer than 2^20 - 1 row
 * tiles (always true for S*k < 2^26): else UNSUPPORTED.
 */
int moe_scatter_ffn_fwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                        const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                        int32_t S, int32_t D, int32_t F, int32_t E, int32_t k, uint16_t *out,
                        void *workspace, size_t workspace_bytes, void *stream);

/*
 * Training-mode forward: moe_scatter_ffn_fwd with the per-route-rows combine
 * that also keeps, for the backward, the gate and up projections a and b of
 * every slot (bf16, rounded from the fp32 sums) and h (as used by the down
 * projection). saved_activations [S*k*3F] bf16, caller-owned: rows [S*k, 2F]
 * holding a in columns [0, F) and b in [F, 2F), followed by h [S*k, F], all
 * in slot order. Passing it to moe_scatter_ffn_bwd skips the backward's
 * recomputation of the gate+up GEMM. out is identical to moe_scatter_ffn_fwd.
 * workspace_bytes >= moe_scatter_ffn_workspace_bytes(); limits as the
 * forward, and S*k*2F < 2^30.
 */
int moe_scatter_ffn_fwd_train(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              int32_t S, int32_t D, int32_t F, int32_t E, int32_t k, uint16_t *out,
                              uint16_t *saved_activations, void *workspace, size_t workspace_bytes, void *stream);

/*
 * Workspace bytes of moe_scatter_ffn_bwd: tile tables, the recomputed
 * a | b [S*k, 2F] and h [S*k, F] (bf16, slot order), slot-order copies of
 * g*dout and x [S*k, D] (bf16), fp32 input-gradient rows [S*k, D] and the
 * router-gate partial sums. Pure host function.
 */
size_t moe_scatter_ffn_bwd_workspace_bytes(int32_t S, int32_t D, int32_t F, int32_t E, int32_t k);

/*
 * Backward of moe_scatter_ffn_fwd (ScatterMoE Guide, "3. Fused Backward Pass
 * Dynamics": input gradients scattered back through W^T to the token rows,
 * weight gradients accumulated per expert; "2. The Hidden Cost of Activation
 * Materialization": the SwiGLU experts). Given dout [S, D] bf16, the
 * gradient of out, and the forward's inputs, with route f = t*k + j of
 * expert e in slot r, g = topk_weights[f], a = x[t] W1[e], b = x[t] W3[e],
 * h = SiLU(a) b (recomputed here, fp32 sums, a and b kept as bf16):
 *   d_topk_weights[f] = <dout[t], h W2[e]>                          fp32 [S, k]
 *   c = dout[t] W2[e]^T;  da = g c b SiLU'(a),  db = g c SiLU(a)    (bf16)
 *   dw2[e] = sum_r h^T (g dout[t])  (g dout[t] rounded to bf16)      fp32 [E, F, D]
 *   dw1[e] = sum_r x[t]^T da,  dw3[e] = sum_r x[t]^T db             fp32 [E, D, F]
 *   dx[t]  = bf16(sum_j da W1[e]^T + db W3[e]^T)  (j in order)       bf16 [S, D]
 * Every weight gradient is reduced on chip per output tile (no atomics);
 * experts with no routes get zero weight gradients; results are
 * reproducible run to run. Any output may be NULL (not all). Arguments,
 * layouts and the map as moe_scatter_ffn_fwd; topk_weights is required.
 * saved_activations: NULL to recompute a, b and h here, or the buffer filled
 * by moe_scatter_ffn_fwd_train for the same inputs (then no recomputation;
 * the gradients are bit-identical); the call overwrites its a | b rows with
 * da | db, so it serves one backward.
 * Limits: D % 64 == 0, F % 64 == 0, E <= 1024, S*D < 2^30, D*F < 2^30,
 * S*k*max(D, 2F) < 2^30 (else UNSUPPORTED).
 */
int moe_scatter_ffn_bwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                        const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                        const uint16_t *dout, int32_t S, int32_t D, int32_t F, int32_t E, int32_t k,
                        uint16_t *saved_activations, uint16_t *dx, float *dw1, float *dw3, float *dw2,
                        float *d_topk_weights, void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_scatter_ffn_bwd with the weight gradients stored in the weights' own
 * dtype: dw1, dw3 [E, D, F] and dw2 [E, F, D] are bf16, each element the
 * fp32 sum of moe_scatter_ffn_bwd rounded once to nearest-even (the same
 * bits as rounding that call's fp32 result). The reduction is unchanged;
 * the stores move half the bytes, which is what bounds the weight-gradient
 * GEMMs of models with many small experts. Everything else (arguments,
 * workspace, limits, saved_activations, NULL outputs) as moe_scatter_ffn_bwd.
 */
int moe_scatter_ffn_bwd_bf16w(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              const uint16_t *dout, int32_t S, int32_t D, int32_t F, int32_t E, int32_t k,
                              uint16_t *saved_activations, uint16_t *dx, uint16_t *dw1, uint16_t *dw3,
                              uint16_t *dw2, float *d_topk_weights, void *workspace, size_t workspace_bytes,
                              void *stream);

/*
 * Workspace bytes of moe_parallel_linear_fwd and moe_parallel_linear_bwd for
 * these sizes (one size serves every grouping mode and both calls): tile
 * tables, fp32 rows [S*k, max(D_in, D_out)] and the bf16 slot-order rows the
 * weight gradient reads. Pure host function.
 */
size_t moe_parallel_linear_workspace_bytes(int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E);

/*
 * ParallelLinear(X, W, I, G) (ScatterMoE Guide, "1. The Anatomy of
 * ParallelLinear" and the figure "The ParallelLinear Core Abstraction": rows
 * of X read by index, multiplied by the routed expert's W, scaled by the
 * router coefficient, with grouped (expert-sorted) or scattered (token
 * order) layouts on either side). With f = t*k + j the route of token t to
 * expert e in slot r (the map of moe_sparse_map):
 *   in(f) = x[r] if grouped_in (x holds S*k rows in slot order),
 *           x[t] otherwise (x holds S token rows, read in place)
 *   z_f   = g_f * in(f) W[e]    (fp32 sums; g_f = gates[f], 1 if gates == NULL)
 *   y[r]  = bf16(z_f)                if grouped_out (y: S*k rows, slot order)
 *   y[t]  = bf16(sum_j z_f)          otherwise (y: S rows; j = 0..k-1 in order,
 *                                    rounded once)
 * w [E, D_in, D_out] bf16 (D_out contiguous); gates [S*k] fp32 or NULL;
 * expert_offsets [E+1] and slot_src [S*k] from moe_sparse_map; grouped_in
 * and grouped_out are 0 or 1. The output is fully written.
 * Limits: D_in % 64 == 0, D_out % 64 == 0, E <= 1024,
 * S*k*max(D_in, D_out) < 2^30, D_in*D_out < 2^30 (else UNSUPPORTED).
 */
int moe_parallel_linear_fwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                            const int32_t *slot_src, int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E,
                            int32_t grouped_in, int32_t grouped_out, uint16_t *y, void *workspace,
                            size_t workspace_bytes, void *stream);

/*
 * Backward of ParallelLinear (ScatterMoE Guide, "3. Fused Backward Pass
 * Dynamics": the input gradient scatters g dY W_e^T back to the rows it came
 * from, the weight gradient accumulates g x^T dY over each expert's tokens).
 * With dy_f = dy[r] if grouped_out, else dy[t] (dy laid out like the
 * forward's y):
 *   dx     [like x]           c_f = dy_f W[e]^T (fp32); dx[r] = bf16(g_f c_f)
 *                             if grouped_in, else dx[t] = bf16(sum_j g_f c_f)
 *   dw     [E, D_in, D_out]   fp32; dw[e] = sum over the slots of expert e of
 *                             in(f)^T (g_f dy_f), the reduction kept on chip
 *                             (one workgroup owns each output tile: no
 *                             atomics); an expert with no routes gets zeros
 *   dgates [S*k]              fp32; dgates[f] = <dy_f, in(f) W[e]>, the
 *                             gradient of the router coefficient
 * Any of dx, dw, dgates may be NULL (not all three). For dw the product
 * g_f * dy_f is rounded to bf16 before the GEMM. Reproducible run to run.
 * Arguments and limits as moe_parallel_linear_fwd; with S == 0 only dw is
 * written (zeros).
 */
int moe_parallel_linear_bwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                            const int32_t *slot_src, const uint16_t *dy, int32_t S, int32_t k, int32_t D_in,
                            int32_t D_out, int32_t E, int32_t grouped_in, int32_t grouped_out, uint16_t *dx,
                            float *dw, float *dgates, void *workspace, size_t workspace_bytes, void *stream);

/*
 * moe_parallel_linear_bwd with dw [E, D_in, D_out] stored as bf16: each
 * element is that call's fp32 sum rounded once to nearest-even. Everything
 * else as moe_parallel_linear_bwd.
 */
int moe_parallel_linear_bwd_bf16w(const uint16_t *x, const uint16_t *w, const float *gates,
                                  const int32_t *expert_offsets, const int32_t *slot_src, const uint16_t *dy,
                                  int32_t S, int32_t k, int32_t D_in, int32_t D_out, int32_t E, int32_t grouped_in,
                                  int32_t grouped_out, uint16_t *dx, uint16_t *dw, float *dgates, void *workspace,
                                  size_t workspace_bytes, void *stream);

/*
 * Profiling hooks (measurement support, not part of the method). While
 * enabled, every kernel launched by the calls above is bracketed by a pair of
 * HIP events recorded on its stream.
 *   moe_profile_start(capacity): create 2*capacity events up front and start
 *     recording (at most `capacity` kernels are recorded; later ones are
 *     not). Clears previous totals.
 *   moe_profile_stop(): stop recording, wait for the recorded events and add
 *     each kernel's elapsed time to its totals.
 *   moe_profile_read(kernel, &name, &total_ms, &launches): totals of kernel
 *     kind `kernel` (0 <= kernel < moe_profile_kinds()); name is a static
 *     string.
 * Host-side state is process-wide and guarded by a mutex.
 */
int moe_profile_start(int capacity);
int moe_profile_stop(void);
int moe_profile_kinds(void);
int moe_profile_read(int kernel, const char **name, double *total_ms, int *launches);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
