// ParallelLinear and its backward.
//
// ScatterMoE Guide, "1. The Anatomy of ParallelLinear" (ParallelLinear(X,
// W, I, G): gathered rows of X times the routed expert's W, scaled by the
// router coefficient, grouped or scattered on either side) and "3. Fused
// Backward Pass Dynamics" (the input gradient scatters g dY W_e^T back to the
// token rows; the weight gradient accumulates g x^T dY per expert).
//
// For route f = t k + j (token t, expert e, gate g_f) in slot r:
//   in(f)  = x[r] (grouped input) or x[t] (scattered input)
//   z_f    = g_f in(f) W[e]
//   y      = z_f at row r (grouped output) or sum_j z_f at row t (scattered)
// Backward, with dy_f = dy[r] (grouped output) or dy[t]:
//   c_f    = dy_f W[e]^T                (input-gradient GEMM, unscaled rows)
//   dx     = g_f c_f at row r, or sum_j g_f c_f at row t     (finalize)
//   dg_f   = <in(f), c_f>  (= <dy_f, in(f) W[e]>)            (finalize)
//   dw[e]  = sum over the expert's slots of in(f)^T (g_f dy_f) (weight GEMM)
//
// Kernels per call (one stream, no host synchronisation):
//   forward   tile table; grouped GEMM (kLinBf16 for grouped output, else
//             kDownRows fp32 rows + ordered combine)
//   backward  tile table; kDownRows GEMM on W^T (dx and/or dg requested);
//             finalize (dx bf16, dg fp32); for dw: the slot-ordered copies
//             the weight GEMM reads (x rows when the input is scattered,
//             g_f dy_f rows unless dy is grouped and ungated), then the
//             grouped weight-gradient GEMM
#include <algorithm>

#include "gemm_pp.hpp"
#include "gemm_wgrad.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

// dst[r] = bf16(g_f * src_row(f)) for slot r, f = slot_src[r]; src_row(f) is
// src[r] when grouped, else src[f / k]; a NULL gate copies the row. Rows of
// D8 x 16 bytes.
__global__ __launch_bounds__(256) void pl_slot_rows_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                           const int32_t *__restrict__ slot_src,
                                                           const float *__restrict__ gate, int n, int k, int D8,
                                                           int grouped) {
    const size_t total = (size_t)n * D8;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const size_t r = i / D8, c = i - r * D8;
        const int f = slot_src[r];
        const size_t srow = grouped ? r : (size_t)(f / k);
        uint4 v = src[srow * D8 + c];
        if (gate) {
            const float g = gate[f];
            uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float lo = bf16_bits_to_f32((uint16_t)(w[q] & 0xffffu)) * g;
                const float hi = bf16_bits_to_f32((uint16_t)(w[q] >> 16)) * g;
                w[q] = (uint32_t)f32_to_bf16_bits(lo) | ((uint32_t)f32_to_bf16_bits(hi) << 16);
            }
            v = make_uint4(w[0], w[1], w[2], w[3]);
        }
        dst[i] = v;
    }
}

// Finalize of the input gradient from the unscaled rows c [S*k, D] (row f):
//   scattered input: one workgroup per token t, routes f = t k + j:
//       dx[t] = bf16(sum_j g_f c_f) (j in order), dg[f] = <x[t], c_f>
//   grouped input: one workgroup per slot r, f = slot_src[r]:
//       dx[r] = bf16(g_f c_f), dg[f] = <x[r], c_f>
// dx or dg may be NULL; a NULL gate means 1. One pass over the rows for up
// to kPlChunk routes per token (more are taken in chunks, dx then in a pass
// of its own); each thread owns fixed groups of 4 columns and the dot
// products are reduced in a fixed order, so results are reproducible.
constexpr int kPlChunk = 16;

__device__ __forceinline__ float pl_block_sum(float v, float *s_w) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) s_w[w] = v;
    __syncthreads();
    return (s_w[0] + s_w[1]) + (s_w[2] + s_w[3]);
}

template <bool GROUPED>
__global__ __launch_bounds__(256) void pl_finalize_kernel(const float4 *__restrict__ c, const uint2 *__restrict__ x,
                                                          const int32_t *__restrict__ slot_src,
                                                          const float *__restrict__ gate, int k, int D4,
                                                          uint2 *__restrict__ dx, float *__restrict__ dg) {
    __shared__ float s_w[4];
    const int item = blockIdx.x;  // token (scattered) or slot (grouped)
    const int nr = GROUPED ? 1 : k;
    const int f0 = GROUPED ? slot_src[item] : item * k;
    const bool fused_dx = dx != nullptr && nr <= kPlChunk;
    const uint2 *xr = x + (size_t)item * D4;
    for (int j0 = 0; j0 < nr; j0 += kPlChunk) {
        const int nj = min(kPlChunk, nr - j0);
        float g[kPlChunk], dot[kPlChunk];
#pragma unroll
        for (int j = 0; j < kPlChunk; ++j) {
            g[j] = (j < nj && gate) ? gate[f0 + j0 + j] : 1.0f;
            dot[j] = 0.f;
        }
        for (int d = threadIdx.x; d < D4; d += 256) {
            const uint2 xv = xr[d];
            const float x0 = bf16_bits_to_f32(xv.x & 0xffffu), x1 = bf16_bits_to_f32(xv.x >> 16);
            const float x2 = bf16_bits_to_f32(xv.y & 0xffffu), x3 = bf16_bits_to_f32(xv.y >> 16);
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
            for (int j = 0; j < kPlChunk; ++j) {
                if (j < nj) {
                    const float4 cv = c[(size_t)(f0 + j0 + j) * D4 + d];
                    s.x += g[j] * cv.x;
                    s.y += g[j] * cv.y;
                    s.z += g[j] * cv.z;
                    s.w += g[j] * cv.w;
                    dot[j] += ((x0 * cv.x + x1 * cv.y) + (x2 * cv.z + x3 * cv.w));
                }
            }
            if (fused_dx) {
                const uint32_t lo = (uint32_t)f32_to_bf16_bits(s.x) | ((uint32_t)f32_to_bf16_bits(s.y) << 16);
                const uint32_t hi = (uint32_t)f32_to_bf16_bits(s.z) | ((uint32_t)f32_to_bf16_bits(s.w) << 16);
                dx[(size_t)item * D4 + d] = make_uint2(lo, hi);
            }
        }
        if (dg) {
#pragma unroll
            for (int j = 0; j < kPlChunk; ++j) {
                if (j < nj) {
                    const float v = pl_block_sum(dot[j], s_w);
                    if (threadIdx.x == 0) dg[f0 + j0 + j] = v;
                }
            }
        }
    }
    if (dx && !fused_dx) {
        for (int d = threadIdx.x; d < D4; d += 256) {
            float4 s = make_float4(0.f, 0.f, 0.f, 0.f);
            for (int j = 0; j < nr; ++j) {
                const float gj = gate ? gate[f0 + j] : 1.0f;
                const float4 cv = c[(size_t)(f0 + j) * D4 + d];
                s.x += gj * cv.x;
                s.y += gj * cv.y;
                s.z += gj * cv.z;
                s.w += gj * cv.w;
            }
            const uint32_t lo = (uint32_t)f32_to_bf16_bits(s.x) | ((uint32_t)f32_to_bf16_bits(s.y) << 16);
            const uint32_t hi = (uint32_t)f32_to_bf16_bits(s.z) | ((uint32_t)f32_to_bf16_bits(s.w) << 16);
            dx[(size_t)item * D4 + d] = make_uint2(lo, hi);
        }
    }
}

// Tile heights of the ParallelLinear GEMMs (one weight matrix, 256-column
// tiles; the forward and input-gradient GEMMs share the height, except the
// grouped-output forward on large experts, see pl_plan): 192
// rows for large experts, 128 rows for ~190-380 rows per expert, 192 rows on
// the short-tile path for ~100-190 (one tile per expert, so its weights
// stream once), then 64 and 32.
static int pl_pick_bm(int64_t avg) {
    if (avg >= 384) return 192;
    if (avg >= 192) return 128;
    if (avg >= 96) return 192;
    if (avg >= 48) return 64;
    return 32;
}

PlPlan pl_plan(int64_t S, int64_t k, int64_t D_in, int64_t D_out, int64_t E) {
    PlPlan pl{};
    const int64_t N = S * k;
    const int64_t avg = N / std::max<int64_t>(E, 1);
    pl.bm = pl_pick_bm(avg);
    pl.bn = pl.bm == 32 ? 128 : 256;
    pl.n_mtiles = tiles_upper_bound(N, E, pl.bm);
    // the grouped-output forward takes 256 x 256 tiles on experts of ~770
    // rows and more (Mixtral up-projection 1.02 -> 0.91 ms); the transposed
    // input-gradient GEMM stays on the shared height (its 256-row instance
    // reloads a spilled DMA offset inside the main loop and is 60 % slower),
    // so the tile table is built per launch
    pl.bm_lin = avg >= 768 ? 256 : pl.bm;
    pl.n_mtiles_lin = tiles_upper_bound(N, E, pl.bm_lin);
    pl.n_ntiles_fwd = (int)((D_out + pl.bn - 1) / pl.bn);
    pl.n_ntiles_dx = (int)((D_in + pl.bn - 1) / pl.bn);
    pl.wg_bm = 256;
    pl.wg_bn = 256;
    pl.wg_mt = (int)((D_in + pl.wg_bm - 1) / pl.wg_bm);
    pl.wg_nt = (int)((D_out + pl.wg_bn - 1) / pl.wg_bn);
    const int nn = std::max(pl.n_ntiles_fwd, pl.n_ntiles_dx);
    size_t off = 0;
    pl.tiles_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles, 1) * sizeof(int4));
    pl.order_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles, 1) * nn * sizeof(uint32_t));
    pl.counts_off = off;
    off += align_up(2 * sizeof(int));
    pl.rows_off = off;  // fp32 rows [S*k, max(D_in, D_out)]
    off += align_up((size_t)N * (size_t)std::max(D_in, D_out) * 4);
    pl.xg_off = off;    // bf16 slot-order input rows [S*k, D_in] (weight gradient)
    off += align_up((size_t)N * (size_t)D_in * 2);
    pl.dyg_off = off;   // bf16 slot-order g * dy rows [S*k, D_out] (weight gradient)
    off += align_up((size_t)N * (size_t)D_out * 2);
    pl.ws_bytes = off;
    return pl;
}

template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A, int FLAGS, bool SKIP = false>
static void launch_pl_tile(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.n_ntiles = (p.N + BN - 1) / BN;
    if (p.n_mtiles * p.n_ntiles == 0) return;
    grouped_gemm_pp_persistent_kernel<BM, BN, MODE, BK, STAGES, STAGES_A, SKIP, FLAGS>
        <<<device_cus(), 512, 0, stream>>>(p);
}

template <int MODE, int FLAGS>
static void launch_pl_gemm(int bm, int64_t avg, const GemmParams &p, hipStream_t stream) {
    switch (bm) {
        case 256:
            // the gate+up tile's ring (3-deep weights, 2-deep rows, DMA
            // shared by the wave groups): Mixtral forward 847-854 -> 811-824
            // us against the 2/2 ring with group 0 issuing
            launch_pl_tile<256, 256, MODE, 64, 3, 2, FLAGS | kFlagSplitDma>(p, stream);
            break;
        case 192:
            // the per-route-rows launches (forward rows, dx) share the DMA
            // issue between the wave groups: dx on Mixtral 889-904 -> 759-763
            // us; on the 256- and 128-row tiles sharing measured 1-5 % slower
            if (avg < 192) launch_pl_tile<192, 256, MODE, 64, 3, 2, FLAGS, true>(p, stream);
            else if constexpr (MODE == kDownRows) launch_pl_tile<192, 256, MODE, 64, 3, 2, FLAGS | kFlagSplitDma, false>(p, stream);
            else launch_pl_tile<192, 256, MODE, 64, 3, 2, FLAGS, false>(p, stream);
            break;
        case 128: launch_pl_tile<128, 256, MODE, 64, 4, 2, FLAGS>(p, stream); break;
        case 64: launch_pl_tile<64, 256, MODE, 64, 3, 3, FLAGS>(p, stream); break;
        default: launch_pl_tile<32, 128, MODE, 64, 4, 4, FLAGS>(p, stream); break;
    }
}

static void pl_tile_table(const PlPlan &pl, char *ws, const int32_t *offsets, int E, int N, int bm, int n_mtiles,
                          int n_ntiles, hipStream_t stream) {
    TileTableArgs ta{};
    int *counts = reinterpret_cast<int *>(ws + pl.counts_off);
    ta.bm[0] = ta.bm[1] = bm;
    ta.n_mtiles[0] = n_mtiles;
    ta.n_mtiles[1] = 0;
    ta.n_ntiles[0] = ta.n_ntiles[1] = n_ntiles;
    ta.tiles[0] = ta.tiles[1] = reinterpret_cast<int4 *>(ws + pl.tiles_off);
    ta.order[0] = ta.order[1] = reinterpret_cast<uint32_t *>(ws + pl.order_off);
    ta.valid[0] = counts;
    ta.valid[1] = counts + 1;  // the unused second class writes its (zero) count here
    launch_tile_table(offsets, E, N, ta, stream);
}

static GemmParams pl_params(const PlPlan &pl, char *ws, const int32_t *slot_src, int k, int N) {
    GemmParams p{};
    p.slot_src = slot_src;
    p.topk = k;
    p.M = N;
    p.tiles = reinterpret_cast<const int4 *>(ws + pl.tiles_off);
    p.order = reinterpret_cast<const uint32_t *>(ws + pl.order_off);
    p.valid_mtiles = reinterpret_cast<const int *>(ws + pl.counts_off);
    p.n_mtiles = pl.n_mtiles;
    return p;
}

hipError_t launch_pl_fwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                         const int32_t *slot_src, int S, int k, int D_in, int D_out, int E, bool grouped_in,
                         bool grouped_out, uint16_t *y, void *workspace, hipStream_t stream) {
    const PlPlan pl = pl_plan(S, k, D_in, D_out, E);
    char *ws = reinterpret_cast<char *>(workspace);
    const int N = S * k;
    const int bm = grouped_out ? pl.bm_lin : pl.bm;
    const int n_mtiles = grouped_out ? pl.n_mtiles_lin : pl.n_mtiles;
    pl_tile_table(pl, ws, expert_offsets, E, N, bm, n_mtiles, pl.n_ntiles_fwd, stream);
    GemmParams p = pl_params(pl, ws, slot_src, k, N);
    p.n_mtiles = n_mtiles;
    p.A = x;
    p.A_rows = grouped_in ? N : S;
    p.gather_a = grouped_in ? 0 : 1;
    p.B0 = w;
    p.gate = gates;
    p.K = D_in;
    p.N = D_out;
    prof_begin(stream, kKPlGemm);
    if (grouped_out) {
        p.C = y;
        launch_pl_gemm<kLinBf16, 0>(bm, (int64_t)N / E, p, stream);
    } else {
        p.C = ws + pl.rows_off;
        launch_pl_gemm<kDownRows, 0>(pl.bm, (int64_t)N / E, p, stream);
    }
    prof_end(stream, kKPlGemm);
    if (!grouped_out) launch_combine_rows(reinterpret_cast<const float *>(ws + pl.rows_off), y, S, D_out, k, stream);
    return hipGetLastError();
}

hipError_t launch_pl_bwd(const uint16_t *x, const uint16_t *w, const float *gates, const int32_t *expert_offsets,
                         const int32_t *slot_src, const uint16_t *dy, int S, int k, int D_in, int D_out, int E,
                         bool grouped_in, bool grouped_out, uint16_t *dx, void *dw, bool dw_bf16, float *dgates,
                         void *workspace, hipStream_t stream) {
    const PlPlan pl = pl_plan(S, k, D_in, D_out, E);
    char *ws = reinterpret_cast<char *>(workspace);
    const int N = S * k;
    if (dx || dgates) {
        pl_tile_table(pl, ws, expert_offsets, E, N, pl.bm, pl.n_mtiles, pl.n_ntiles_dx, stream);
        // c_f = dy_f W[e]^T, unscaled, fp32 at row f
        GemmParams p = pl_params(pl, ws, slot_src, k, N);
        p.A = dy;
        p.A_rows = grouped_out ? N : S;
        p.gather_a = grouped_out ? 0 : 1;
        p.B0 = w;
        p.gate = nullptr;
        p.K = D_out;
        p.N = D_in;
        p.C = ws + pl.rows_off;
        prof_begin(stream, kKPlDxGemm);
        launch_pl_gemm<kDownRows, kFlagBT>(pl.bm, (int64_t)N / E, p, stream);
        prof_end(stream, kKPlDxGemm);
        const float4 *c = reinterpret_cast<const float4 *>(ws + pl.rows_off);
        const uint2 *x4 = reinterpret_cast<const uint2 *>(x);
        uint2 *dx4 = reinterpret_cast<uint2 *>(dx);
        prof_begin(stream, kKPlFinalize);
        if (grouped_in) {
            if (N > 0) pl_finalize_kernel<true><<<N, 256, 0, stream>>>(c, x4, slot_src, gates, k, D_in / 4, dx4, dgates);
        } else {
            if (S > 0) pl_finalize_kernel<false><<<S, 256, 0, stream>>>(c, x4, slot_src, gates, k, D_in / 4, dx4, dgates);
        }
        prof_end(stream, kKPlFinalize);
    }
    if (dw) {
        const uint16_t *a = x;
        const uint16_t *b = dy;
        prof_begin(stream, kKPlPrep);
        if (!grouped_in) {
            uint16_t *xg = reinterpret_cast<uint16_t *>(ws + pl.xg_off);
            const size_t n8 = (size_t)N * (D_in / 8);
            pl_slot_rows_kernel<<<grid_for(n8, 256 * 4), 256, 0, stream>>>(
                reinterpret_cast<const uint4 *>(x), reinterpret_cast<uint4 *>(xg), slot_src, nullptr, N, k, D_in / 8, 0);
            a = xg;
        }
        if (!grouped_out || gates) {
            uint16_t *dyg = reinterpret_cast<uint16_t *>(ws + pl.dyg_off);
            const size_t n8 = (size_t)N * (D_out / 8);
            pl_slot_rows_kernel<<<grid_for(n8, 256 * 4), 256, 0, stream>>>(
                reinterpret_cast<const uint4 *>(dy), reinterpret_cast<uint4 *>(dyg), slot_src, gates, N, k,
                D_out / 8, grouped_out ? 1 : 0);
            b = dyg;
        }
        prof_end(stream, kKPlPrep);
        WgradParams q{};
        q.A = a;
        q.B0 = b;
        q.B1 = nullptr;
        q.offsets = expert_offsets;
        q.C0 = dw;
        q.out_bf16 = dw_bf16;
        q.C1 = nullptr;
        q.M = D_in;
        q.N = D_out;
        q.ldb = D_out;
        q.E = E;
        q.n_mt = pl.wg_mt;
        q.n_nt = pl.wg_nt;
        prof_begin(stream, kKPlWgrad);
        launch_grouped_wgrad<256, 256, 1>(q, N, E, device_cus(), stream);
        prof_end(stream, kKPlWgrad);
    }
    return hipGetLastError();
}

}  // namespace smoe
