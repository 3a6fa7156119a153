// Backward of the scattered SwiGLU expert FFN with weighted combine.
//
// ScatterMoE Guide, "3. Fused Backward Pass Dynamics" (input gradient
// scattered back through W^T to the token rows, weight gradient accumulated
// per expert on chip) applied to both expert linears, with the SwiGLU and the
// router coefficient between them. For route f = t k + j (expert e, gate g)
// in slot r, with a = x W1[e], b = x W3[e], h = SiLU(a) b:
//   dg[f]   = <dout[t], h W2[e]> = <h, c>,   c = dout[t] W2[e]^T
//   da, db  = g c b SiLU'(a),  g c SiLU(a)
//   dW2[e]  = sum_r h^T (g dout[t]),   dW1[e], dW3[e] = sum_r x^T da, x^T db
//   dx[t]   = sum_j da W1[e]^T + db W3[e]^T
//
// Kernels (one stream, no host synchronisation):
//   tile tables     the expert tiles and block orders of the four GEMMs
//   recompute       gate+up GEMM saving a, b (bf16, [S*k, 2F]) and h (skipped
//                   when the training-mode forward kept them)
//   slot rows       g dout[t] and x[t] copied to slot order (weight GEMMs)
//   dh              W2^T GEMM of the gathered dout rows; its epilogue turns
//                   a, b into da, db in place and writes <h, c> partials
//   gate reduce     dg[f] = sum of the partials in a fixed order
//   dW2             weight-gradient GEMM h^T (g dout)
//   dW1, dW3        one weight-gradient GEMM, x^T [da | db]
//   dx              [da | db] [W1 ; W3]^T (K split over the two weights),
//                   per-route fp32 rows, then the ordered combine
#include <algorithm>

#include "gemm_pp.hpp"
#include "gemm_wgrad.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

__global__ __launch_bounds__(256) void ffn_bwd_slot_rows_kernel(const uint4 *__restrict__ src, uint4 *__restrict__ dst,
                                                                const int32_t *__restrict__ slot_src,
                                                                const float *__restrict__ gate, int n, int k, int D8) {
    const size_t total = (size_t)n * D8;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const size_t r = i / D8, c = i - r * D8;
        const int f = slot_src[r];
        uint4 v = src[(size_t)(f / k) * D8 + c];
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

// dg[f] = sum over p of part[p * n + f]: a workgroup takes 64 routes (one per
// lane); wave w sums the partials p = w, w + 4, ... in order and the four
// wave sums are added in a fixed order, so the result is reproducible.
__global__ __launch_bounds__(256) void ffn_bwd_gate_reduce_kernel(const float *__restrict__ part, int nparts, int n,
                                                                  float *__restrict__ dg) {
    __shared__ float s_w[4][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int f = blockIdx.x * 64 + lane;
    float s = 0.f;
    if (f < n)
        for (int q = w; q < nparts; q += 4) s += part[(size_t)q * n + f];
    s_w[w][lane] = s;
    __syncthreads();
    if (w == 0 && f < n) dg[f] = (s_w[0][lane] + s_w[1][lane]) + (s_w[2][lane] + s_w[3][lane]);
}

// Tile rows of the dh GEMM: 192 for experts of ~100-190 rows (one tile per
// expert, so its W2 streams once; the short-tile path skips missing rows)
// and, since the 192-row tile shares its DMA issue between the wave groups,
// for experts of 384 rows and more (Mixtral dh 1095-1110 -> 1076-1081 us,
// Qwen2 S = 4096 811-822 -> 726-740 us against 128-row tiles); else 128 / 64
// / 32.
static int bwd_pick_bm(int64_t avg) {
    if (avg >= 384) return 192;
    if (avg >= 192) return 128;
    if (avg >= 96) return 192;
    if (avg >= 48) return 64;
    return 32;
}

// The input-gradient GEMM (K = 2F) takes 192-row tiles once experts are
// large (measured on Mixtral: 1.82 against 2.13 ms with 128-row tiles); from
// 192 to 383 rows per expert it keeps 128-row tiles (GPT-OSS dx 1388-1390
// against 1508-1514 us with 192 rows).
static int bwd_pick_bm_dx(int64_t avg) { return avg >= 384 ? 192 : bwd_pick_bm(avg); }

FfnBwdPlan ffn_bwd_plan(int64_t S, int64_t D, int64_t F, int64_t E, int64_t k) {
    FfnBwdPlan pl{};
    const int64_t N = S * k;
    const int64_t avg = N / std::max<int64_t>(E, 1);
    pl.bm_r = pick_bm(avg);
    pl.bm_b = bwd_pick_bm(avg);
    pl.bm_x = bwd_pick_bm_dx(avg);
    pl.bn_b = pl.bm_b == 32 ? 128 : 256;
    const int bn_x = pl.bm_x == 32 ? 128 : 256;
    pl.nm_r = tiles_upper_bound(N, E, pl.bm_r);
    pl.nm_b = tiles_upper_bound(N, E, pl.bm_b);
    pl.nm_x = tiles_upper_bound(N, E, pl.bm_x);
    pl.nn_r = (int)((F + 127) / 128);
    pl.nn_h = (int)((F + pl.bn_b - 1) / pl.bn_b);
    pl.nn_x = (int)((D + bn_x - 1) / bn_x);
    pl.nparts = pl.nn_h;  // one <h, c> partial per column tile of the dh GEMM and route
    size_t off = 0;
    auto take = [&](size_t bytes) {
        const size_t o = off;
        off += align_up(std::max<size_t>(bytes, 1));
        return o;
    };
    pl.tiles_r = take((size_t)pl.nm_r * sizeof(int4));
    pl.tiles_b = take((size_t)pl.nm_b * sizeof(int4));
    pl.tiles_x = take((size_t)pl.nm_x * sizeof(int4));
    pl.order_r = take((size_t)pl.nm_r * pl.nn_r * 4);
    pl.order_h = take((size_t)pl.nm_b * pl.nn_h * 4);
    pl.order_x = take((size_t)pl.nm_x * pl.nn_x * 4);
    pl.counts = take(4 * sizeof(int));
    pl.ab = take((size_t)N * 2 * F * 2);
    pl.h = take((size_t)N * F * 2);
    pl.dyg = take((size_t)N * D * 2);
    pl.xg = take((size_t)N * D * 2);
    pl.rows = take((size_t)N * D * 4);
    pl.part = take((size_t)pl.nparts * N * 4);
    pl.ws_bytes = off;
    return pl;
}

template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A, bool SKIP, int FLAGS>
static void bwd_tile(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.n_ntiles = (p.N + BN - 1) / BN;
    if (p.n_mtiles * p.n_ntiles == 0) return;
    grouped_gemm_pp_persistent_kernel<BM, BN, MODE, BK, STAGES, STAGES_A, SKIP, FLAGS>
        <<<device_cus(), 512, 0, stream>>>(p);
}

// gate+up recomputation: the tile shapes of the forward gate+up GEMM, with
// its 3-deep weight ring; below ~770 rows per expert, as in the forward, the
// short-tile form over evenly split tiles (GPT-OSS recomputation 1469-1497
// -> 1352-1375 us, Qwen2 S = 4096 1288-1338 -> 1233-1274 us against the
// plain 2-deep form)
static void launch_recompute(int bm, int64_t avg, const GemmParams &p, hipStream_t stream) {
    switch (bm) {
        case 256:
            if (avg >= 768) bwd_tile<256, 128, kGateUpSave, 64, 3, 2, false, 0>(p, stream);
            else bwd_tile<256, 128, kGateUpSave, 64, 3, 2, true, 0>(p, stream);
            break;
        case 192: bwd_tile<192, 128, kGateUpSave, 64, 3, 2, true, 0>(p, stream); break;
        case 64: bwd_tile<64, 128, kGateUpSave, 64, 3, 3, false, 0>(p, stream); break;
        default: bwd_tile<32, 128, kGateUpSave, 64, 4, 4, false, 0>(p, stream); break;
    }
}

// one transposed weight, 256-column tiles (128 for 32-row tiles); 192-row
// tiles over experts shorter than the tile take the short-tile path. The
// 192-row plain tiles and the 128-row tiles share the DMA issue between the
// two wave groups (two alternating runs on one box: dx on Mixtral 1800-1803 ->
// 1496-1510 us, Qwen2 S = 4096 1239-1263 -> 1156-1159 us; dh on Mixtral
// 1156-1165 -> 1101-1103 us, Qwen2 843-860 -> 820-825 us, GPT-OSS 929-947 ->
// 913-918 us; GPT-OSS dx unchanged)
template <int MODE, int FLAGS>
static void launch_bwd_bt(int bm, int64_t avg, const GemmParams &p, hipStream_t stream) {
    switch (bm) {
        case 192:
            if (avg < 192) bwd_tile<192, 256, MODE, 64, 3, 2, true, FLAGS>(p, stream);
            else bwd_tile<192, 256, MODE, 64, 3, 2, false, FLAGS | kFlagSplitDma>(p, stream);
            break;
        case 128: bwd_tile<128, 256, MODE, 64, 4, 2, false, FLAGS | kFlagSplitDma>(p, stream); break;
        case 64: bwd_tile<64, 256, MODE, 64, 3, 3, false, FLAGS>(p, stream); break;
        default: bwd_tile<32, 128, MODE, 64, 4, 4, false, FLAGS>(p, stream); break;
    }
}

hipError_t launch_ffn_bwd(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                          const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                          const uint16_t *dout, int S, int D, int F, int E, int k, uint16_t *saved, uint16_t *dx,
                          void *dw1, void *dw3, void *dw2, bool dw_bf16, float *dg, void *workspace,
                          hipStream_t stream) {
    const FfnBwdPlan pl = ffn_bwd_plan(S, D, F, E, k);
    char *ws = reinterpret_cast<char *>(workspace);
    const int N = S * k;
    int *counts = reinterpret_cast<int *>(ws + pl.counts);
    int4 *tiles_r = reinterpret_cast<int4 *>(ws + pl.tiles_r);
    int4 *tiles_b = reinterpret_cast<int4 *>(ws + pl.tiles_b);
    int4 *tiles_x = reinterpret_cast<int4 *>(ws + pl.tiles_x);
    // a | b and h: saved by the training-mode forward, else recomputed here
    uint16_t *ab = saved ? saved : reinterpret_cast<uint16_t *>(ws + pl.ab);
    uint16_t *h = saved ? saved + (size_t)N * 2 * F : reinterpret_cast<uint16_t *>(ws + pl.h);
    uint16_t *dyg = reinterpret_cast<uint16_t *>(ws + pl.dyg);
    uint16_t *xg = reinterpret_cast<uint16_t *>(ws + pl.xg);
    float *rows = reinterpret_cast<float *>(ws + pl.rows);
    float *part = reinterpret_cast<float *>(ws + pl.part);

    TileTableArgs ta{};
    ta.bm[0] = pl.bm_r;
    ta.n_mtiles[0] = pl.nm_r;
    ta.n_ntiles[0] = pl.nn_r;
    ta.tiles[0] = tiles_r;
    ta.order[0] = reinterpret_cast<uint32_t *>(ws + pl.order_r);
    ta.valid[0] = counts;
    ta.bm[1] = pl.bm_b;
    ta.n_mtiles[1] = pl.nm_b;
    ta.n_ntiles[1] = pl.nn_h;
    ta.tiles[1] = tiles_b;
    ta.order[1] = reinterpret_cast<uint32_t *>(ws + pl.order_h);
    ta.valid[1] = counts + 1;
    ta.split[0] = (pl.bm_r == 256 && (int64_t)N / std::max(E, 1) < 768);  // as the forward's short-tile launches
    launch_tile_table(expert_offsets, E, N, ta, stream);
    TileTableArgs tx{};
    tx.bm[0] = tx.bm[1] = pl.bm_x;
    tx.n_mtiles[0] = pl.nm_x;
    tx.n_mtiles[1] = 0;
    tx.n_ntiles[0] = tx.n_ntiles[1] = pl.nn_x;
    tx.tiles[0] = tx.tiles[1] = tiles_x;
    tx.order[0] = tx.order[1] = reinterpret_cast<uint32_t *>(ws + pl.order_x);
    tx.valid[0] = counts + 2;
    tx.valid[1] = counts + 3;
    launch_tile_table(expert_offsets, E, N, tx, stream);

    GemmParams p{};
    p.slot_src = slot_src;
    p.topk = k;
    p.M = N;
    p.A_rows = S;

    // a, b and h of every slot
    p.tiles = tiles_r;
    p.order = reinterpret_cast<const uint32_t *>(ws + pl.order_r);
    p.valid_mtiles = counts;
    p.n_mtiles = pl.nm_r;
    p.A = x;
    p.B0 = w1;
    p.B1 = w3;
    p.C = ab;
    p.C2 = h;
    p.N = F;
    p.K = D;
    if (!saved) {
        prof_begin(stream, kKBwdRecompute);
        launch_recompute(pl.bm_r, (int64_t)N / std::max(E, 1), p, stream);
        prof_end(stream, kKBwdRecompute);
    }

    // c = dout[t] W2[e]^T; epilogue: da, db over a, b and the <h, c> partials
    p.tiles = tiles_b;
    p.order = reinterpret_cast<const uint32_t *>(ws + pl.order_h);
    p.valid_mtiles = counts + 1;
    p.n_mtiles = pl.nm_b;
    p.A = dout;
    p.gather_a = 1;
    p.B0 = w2;
    p.B1 = nullptr;
    p.C = ab;
    p.C2 = nullptr;
    p.gate = topk_weights;
    p.part = part;
    p.N = F;
    p.K = D;
    prof_begin(stream, kKBwdDh);
    launch_bwd_bt<kSwigluBwd, kFlagBT>(pl.bm_b, (int64_t)N / E, p, stream);
    prof_end(stream, kKBwdDh);

    if (dg && N > 0) {  // S == 0 with a weight gradient requested reaches here: no routes, empty grid
        prof_begin(stream, kKBwdPrep);
        ffn_bwd_gate_reduce_kernel<<<(N + 63) / 64, 256, 0, stream>>>(part, pl.nparts, N, dg);
        prof_end(stream, kKBwdPrep);
    }

    if (dw2 || dw1 || dw3) {
        prof_begin(stream, kKBwdPrep);
        const size_t n8 = (size_t)N * (D / 8);
        if (dw2)
            ffn_bwd_slot_rows_kernel<<<grid_for(n8, 256 * 4), 256, 0, stream>>>(
                reinterpret_cast<const uint4 *>(dout), reinterpret_cast<uint4 *>(dyg), slot_src, topk_weights, N, k,
                D / 8);
        if (dw1 || dw3)
            ffn_bwd_slot_rows_kernel<<<grid_for(n8, 256 * 4), 256, 0, stream>>>(
                reinterpret_cast<const uint4 *>(x), reinterpret_cast<uint4 *>(xg), slot_src, nullptr, N, k, D / 8);
        prof_end(stream, kKBwdPrep);
    }
    if (dw2) {
        WgradParams q{};
        q.A = h;
        q.B0 = dyg;
        q.offsets = expert_offsets;
        q.C0 = dw2;
        q.out_bf16 = dw_bf16;
        q.M = F;
        q.N = D;
        q.E = E;
        q.ldb = D;
        q.n_mt = (F + 255) / 256;
        q.n_nt = (D + 255) / 256;
        prof_begin(stream, kKBwdWgrad);
        launch_grouped_wgrad<256, 256, 1>(q, N, E, device_cus(), stream);
        prof_end(stream, kKBwdWgrad);
    }
    if (dw1 || dw3) {
        // both from one pass over x (dw1 or dw3 NULL: that half is written to the other's buffer first)
        WgradParams q{};
        q.A = xg;
        q.B0 = ab;
        q.B1 = ab + F;
        q.offsets = expert_offsets;
        q.C0 = dw1 ? dw1 : dw3;
        q.C1 = dw3 ? dw3 : dw1;
        q.out_bf16 = dw_bf16;
        q.M = D;
        q.N = F;
        q.E = E;
        q.ldb = 2 * F;
        q.n_mt = (D + 255) / 256;
        q.n_nt = (F + 127) / 128;
        if (!dw1) q.B0 = ab + F;   // only dw3: both halves compute x^T db
        if (!dw3) q.B1 = ab;       // only dw1: both halves compute x^T da
        prof_begin(stream, kKBwdWgrad);
        launch_grouped_wgrad<256, 128, 2>(q, N, E, device_cus(), stream);
        prof_end(stream, kKBwdWgrad);
    }

    if (dx) {
        // [da | db] [W1 ; W3]^T per route (fp32 rows), then the ordered combine
        p.tiles = tiles_x;
        p.order = reinterpret_cast<const uint32_t *>(ws + pl.order_x);
        p.valid_mtiles = counts + 2;
        p.n_mtiles = pl.nm_x;
        p.A = ab;
        p.gather_a = 0;
        p.B0 = w1;
        p.B1 = w3;
        p.C = rows;
        p.gate = nullptr;
        p.part = nullptr;
        p.N = D;
        p.K = 2 * F;
        prof_begin(stream, kKBwdDx);
        launch_bwd_bt<kDownRows, kFlagBT | kFlagKSplit>(pl.bm_x, (int64_t)N / E, p, stream);
        prof_end(stream, kKBwdDx);
        launch_combine_rows(rows, dx, S, D, k, stream);
    }
    return hipGetLastError();
}

}  // namespace smoe
