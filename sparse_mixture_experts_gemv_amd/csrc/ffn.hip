// Scattered SwiGLU expert FFN with router-weighted scatter-add combine.
//
// ScatterMoE Guide, "The ParallelLinear Core Abstraction" and "1. The
// Anatomy of ParallelLinear": token rows are read in place through the
// expert-sorted index (no [S*k, D] copy), each expert's rows are cut into
// ceil(N_e / BM) tiles with a masked last tile (no padding), the expert GEMM
// runs per tile and the result is scaled by the router coefficient and
// accumulated into the token's output row.
//
// Launch sequence on one stream (no host synchronisation), default combine:
//   tile_table  expert offsets -> (expert, row_begin, row_end) per M tile
//   gate+up     h[r] = bf16(SiLU(x[t] W1[e]) * (x[t] W3[e]))  (gathered A)
//   down        y[f] = w_f * (h[r] W2[e])        (fp32 row f of a per-route buffer)
//   combine     out[t] = bf16(sum_j y[t k + j])   (j = 0 .. k-1 in order)
// Atomic combine (smaller workspace): acc_zero (fp32 [S, D] = 0), gate+up,
// down with acc[t] += w_f * (h[r] W2[e]) by fp32 atomics, finalize
// out = bf16(acc).
#include <algorithm>

#include "gemm.hpp"
#include "gemm_pp.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

// One thread per expert computes ceil(rows / bm) tiles, an exclusive scan
// gives each expert its first tile T_e, and (in workgroup 0) the expert
// writes its (expert, row_begin, row_end) entries: bm rows per tile and the
// rest in the last, or (split) the rows shared evenly over the same number
// of tiles, so that no tile of the expert is much shorter than the others.
// The block order is then filled by the threads of every workgroup, each
// workgroup having formed the same T_e: blocks [T_e * nn, (T_e + c_e) * nn)
// belong to expert e (c_e its tile count, nn the N tiles), N tile major, the
// expert's M tiles minor; a thread finds the expert of a block by binary
// search over T_e. Two GEMMs (tile heights) are handled in one launch.
// Entries past the real tile count are marked empty (expert = -1, order M
// field all ones).
__global__ __launch_bounds__(1024) void tile_table_kernel(const int32_t *__restrict__ offsets, int E, int N,
                                                          const TileTableArgs a) {
    __shared__ int s_wave[2][16];
    __shared__ int s_first[2][1025];  // T_e, with T_E = total
    const int e = threadIdx.x;
    const int lane = e & 63, w = e >> 6;
    int off = 0, end = 0;
    if (e < E) {
        off = min(max(offsets[e], 0), N);
        end = min(max(offsets[e + 1], off), N);
    }
    int t[2], x[2];
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        t[q] = (e < E) ? (end - off + a.bm[q] - 1) / a.bm[q] : 0;
        x[q] = t[q];
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const int y = __shfl_up(x[q], d);
            if (lane >= d) x[q] += y;
        }
        if (lane == 63) s_wave[q][w] = x[q];
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        int base = 0, total = 0;
        for (int i = 0; i < 16; ++i) {
            if (i < w) base += s_wave[q][i];
            total += s_wave[q][i];
        }
        base += x[q] - t[q];
        const int nm = a.n_mtiles[q];
        const int valid = min(total, nm);
        if (e < E) s_first[q][e] = min(base, valid);
        if (e == 0) {
            s_first[q][E] = valid;
            if (blockIdx.x == 0) *a.valid[q] = valid;
        }
        if (blockIdx.x == 0) {
            const int cnt = min(t[q], max(nm - base, 0));
            // even split: the first `extra` tiles hold one row more than the rest
            const int rows = end - off;
            const bool even = a.split[q] && t[q] > 0;
            const int h = even ? rows / t[q] : a.bm[q];
            const int extra = even ? rows - h * t[q] : 0;
            for (int i = 0; i < cnt; ++i) {
                const int r0 = i * h + min(i, extra);
                const int r1 = min(r0 + h + (i < extra ? 1 : 0), rows);
                a.tiles[q][base + i] = make_int4(e, off + r0, off + r1, 0);
            }
            for (int j = valid + threadIdx.x; j < nm; j += 1024) a.tiles[q][j] = make_int4(-1, 0, 0, 0);
            if (a.queue[q] && threadIdx.x < kQueueInts) a.queue[q][threadIdx.x] = 0;
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int nm = a.n_mtiles[q], nn = a.n_ntiles[q];
        const int valid = s_first[q][E];
        const size_t vblocks = (size_t)valid * nn;
        for (size_t L = (size_t)blockIdx.x * 1024 + threadIdx.x; L < (size_t)nm * nn; L += (size_t)gridDim.x * 1024) {
            uint32_t v = kOrderMtMask;
            if (L < vblocks) {
                // expert: the last e with T_e * nn <= L (experts with no tiles share T_e)
                int lo = 0, hi = E - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) >> 1;
                    if ((size_t)s_first[q][mid] * nn <= L) lo = mid;
                    else hi = mid - 1;
                }
                const int first = s_first[q][lo];
                const int cnt = s_first[q][lo + 1] - first;
                const int idx = (int)(L - (size_t)first * nn);
                v = (uint32_t)(first + idx % cnt) | ((uint32_t)(idx / cnt) << kOrderMtBits);
            }
            a.order[q][L] = v;
        }
    }
}

__global__ __launch_bounds__(256) void acc_zero_kernel(float4 *__restrict__ acc, size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride)
        acc[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void acc_finalize_kernel(const float4 *__restrict__ acc, uint2 *__restrict__ out,
                                                           size_t n4) {
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const float4 v = acc[i];
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
        out[i] = make_uint2(lo, hi);
    }
}

// out[t, :] = bf16(sum_j y[t k + j, :]) for the per-route rows y (route f =
// t k + j keeps the k rows of a token adjacent); the k terms are added in
// the order j = 0 .. k-1, so the result does not depend on scheduling.
__global__ __launch_bounds__(256) void combine_rows_kernel(const float4 *__restrict__ y, uint2 *__restrict__ out,
                                                           int S, int D4, int k) {
    const size_t n4 = (size_t)S * D4;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        const size_t t = i / D4, c = i - t * D4;
        const float4 *src = y + t * k * D4 + c;
        float4 v = src[0];
        for (int j = 1; j < k; ++j) {
            const float4 u = src[(size_t)j * D4];
            v.x += u.x;
            v.y += u.y;
            v.z += u.z;
            v.w += u.w;
        }
        const uint32_t lo = (uint32_t)f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16);
        out[i] = make_uint2(lo, hi);
    }
}

void launch_tile_table(const int32_t *offsets, int E, int N, const TileTableArgs &a, hipStream_t stream) {
    prof_begin(stream, kKTileTable);
    // one workgroup per 1024 order entries of the larger table (at most 64):
    // each thread then fills about one entry per table (measured against
    // 4096 entries per workgroup: 12.8 -> 9.7 us on Qwen2 S = 4096, 12.1 ->
    // 8.9 us on DS-V3)
    const size_t entries = std::max((size_t)a.n_mtiles[0] * a.n_ntiles[0], (size_t)a.n_mtiles[1] * a.n_ntiles[1]);
    const int grid = (int)std::min<size_t>(64, std::max<size_t>(1, (entries + 1023) / 1024));
    tile_table_kernel<<<grid, 1024, 0, stream>>>(offsets, E, N, a);
    prof_end(stream, kKTileTable);
}

void launch_combine_rows(const float *y, uint16_t *out, int S, int D, int k, hipStream_t stream) {
    const size_t n4 = (size_t)S * D / 4;
    prof_begin(stream, kKCombine);
    // one float4 per thread where the grid allows it: with few tokens the
    // k loads of a thread are its whole latency chain
    combine_rows_kernel<<<grid_for(n4, 256), 256, 0, stream>>>(reinterpret_cast<const float4 *>(y),
                                                                    reinterpret_cast<uint2 *>(out), S, D / 4, k);
    prof_end(stream, kKCombine);
}

// Tile height per GEMM from the mean rows per expert (known on the host
// without reading the device-side counts): 256 rows from 192 up, 192 rows
// from 96 (an expert of ~128 +- 3 sigma rows fits one tile, so its weights
// stream once), 64 rows from 48, else 32 rows (decode-sized batches: the
// weights dominate and a shallow tile keeps the MFMA work small).
int pick_bm(int64_t avg) {
    if (avg >= 192) return 256;
    if (avg >= 96) return 192;
    if (avg >= 48) return 64;
    return 32;
}

// The down GEMM has few column tiles (D / 256), so its tile count is small
// and the last round of the persistent grid can run half empty; its tile
// height is chosen separately (measured on the five workloads): 128 rows
// with 64-deep k-steps for ~190-380 rows per expert, 192 rows above that and
// for ~100-190 rows per expert.
static int pick_bm_down(int64_t avg) {
    if (avg >= 192 && avg < 384) return 128;
    if (avg >= 96) return 192;
    return pick_bm(avg);
}

int tiles_upper_bound(int64_t N, int64_t E, int bm) {
    return (int)((N + std::min(E, N) * (bm - 1)) / bm);
}

FfnPlan ffn_plan(int64_t S, int64_t D, int64_t F, int64_t E, int64_t k, bool atomic) {
    FfnPlan pl;
    pl.atomic = atomic;
    const int64_t N = S * k;
    const int64_t avg = N / std::max<int64_t>(E, 1);
    pl.bm_up = pick_bm(avg);
    pl.bm_down = pick_bm_down(avg);
    pl.n_mtiles_up = tiles_upper_bound(N, E, pl.bm_up);
    pl.n_mtiles_down = tiles_upper_bound(N, E, pl.bm_down);
    pl.bn_up = 128;
    pl.bn_down = (pl.bm_down == 32) ? 128 : 256;
    pl.n_ntiles_up = (int)((F + pl.bn_up - 1) / pl.bn_up);
    pl.n_ntiles_down = (int)((D + pl.bn_down - 1) / pl.bn_down);
    size_t off = 0;
    pl.tiles_up_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles_up, 1) * sizeof(int4));
    pl.tiles_down_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles_down, 1) * sizeof(int4));
    pl.order_up_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles_up, 1) * pl.n_ntiles_up * sizeof(uint32_t));
    pl.order_down_off = off;
    off += align_up((size_t)std::max(pl.n_mtiles_down, 1) * pl.n_ntiles_down * sizeof(uint32_t));
    pl.counts_off = off;
    off += align_up(2 * sizeof(int));
    pl.queue_off = off;
    off += align_up(kQueueInts * sizeof(int));
    pl.h_off = off;
    off += align_up((size_t)N * (size_t)F * 2);
    pl.acc_off = off;
    off += align_up((size_t)(atomic ? S : S * k) * (size_t)D * 4);
    pl.ws_bytes = off;
    return pl;
}

int grid_for(size_t n, int per_block) {
    const size_t b = (n + per_block - 1) / per_block;
    return (int)std::min<size_t>(std::max<size_t>(b, 1), 2048);
}

int device_cus() {
    static int cached[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cached[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cached[dev] = n;
    }
    return cached[dev];
}

// Gate+up and per-route-rows down GEMMs: one persistent workgroup per CU
// walking whole tiles of the block order (plain-store epilogues, so tiles are
// never split); a tile's epilogue overlaps the next tile's first loads. The
// gate+up GEMM claims its tiles from the per-XCD queues; the down GEMM walks
// the order statically (measured, the queue made it 1-3 % slower on the
// five workloads, while the gate+up gained up to 3 %).
template <int BM, int BN, int MODE, int BK, int STAGES, int STAGES_A = STAGES, bool SKIP_ROWS = false, int FLAGS = 0>
static void launch_pp_persistent(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.n_ntiles = (p.N + BN - 1) / BN;
    if (p.n_mtiles * p.n_ntiles == 0) return;
    constexpr bool kQueue = (MODE == kGateUp || MODE == kGateUpSave);
    grouped_gemm_pp_persistent_kernel<BM, BN, MODE, BK, STAGES, STAGES_A, SKIP_ROWS, FLAGS, kQueue>
        <<<device_cus(), 512, 0, stream>>>(p);
}

// Stream-K down GEMM: one persistent workgroup per CU (160 KB of LDS each).
template <int BM, int BN, int BK, int STAGES>
static void launch_pp_streamk(const GemmParams &p0, hipStream_t stream) {
    GemmParams p = p0;
    p.n_ntiles = (p.N + BN - 1) / BN;
    if (p.n_mtiles * p.n_ntiles == 0) return;
    grouped_gemm_pp_streamk_kernel<BM, BN, BK, STAGES><<<device_cus(), 512, 0, stream>>>(p);
}

// From this many mean rows per expert the 256-row gate+up tiles run the
// plain loop; below it, the short-tile form, and each expert's rows are
// shared evenly over its tiles (tiles of one expert then take about the
// same time, so those sharing a weight panel stay in step; measured on
// GPT-OSS: gate+up 1339 -> 1315-1323 us). Both use a 3-deep weight ring.
constexpr int64_t kUpPlainRows = 768;

// avg = mean rows per expert. Where it is below the tile height (experts of
// ~100-190 rows under 192-row tiles) most tiles are short, so those launches
// skip the MFMAs and row loads of missing rows.
template <int MODE>
static void launch_gemm(int bm, int64_t avg, const GemmParams &p, hipStream_t stream) {
    const int kid = (MODE == kGateUp || MODE == kGateUpSave) ? kKGateUp : kKDown;
    prof_begin(stream, kid);
    if constexpr (MODE == kGateUp || MODE == kGateUpSave) {
        switch (bm) {
            case 256:
                // short tiles skip missing rows where they are common; with
                // ~1000 rows per expert the plain loop keeps the workgroups
                // sharing a weight panel in step (half the HBM re-reads).
                // The weight ring is 3 deep (two k-steps of weights in
                // flight, the LDS full at 160 KB): with the even split, the
                // short-tile launches gained 4.5 % (GPT-OSS) and 3.7 % (Qwen2
                // S = 4096) over a 2-deep ring
                if (avg < kUpPlainRows) launch_pp_persistent<256, 128, MODE, 64, 3, 2, true>(p, stream);
                else launch_pp_persistent<256, 128, MODE, 64, 3, 2>(p, stream);
                break;
            case 192: launch_pp_persistent<192, 128, MODE, 64, 3, 2, true>(p, stream); break;
            case 64: launch_pp_persistent<64, 128, MODE, 64, 3>(p, stream); break;
            default: launch_pp_persistent<32, 128, MODE, 64, 4>(p, stream); break;
        }
    } else if constexpr (MODE == kDown) {
        switch (bm) {
            case 192: launch_pp_streamk<192, 256, 32, 5>(p, stream); break;
            case 128: launch_pp_streamk<128, 256, 64, 3>(p, stream); break;
            case 64: launch_pp_streamk<64, 256, 64, 3>(p, stream); break;
            default: launch_pp_streamk<32, 128, 64, 4>(p, stream); break;
        }
    } else {
        switch (bm) {
            case 192:
                // 64-deep k-steps in a 3/2 ring with the two wave groups
                // sharing the DMA issue: Mixtral 907-912 -> 858-863 us and
                // Qwen2 S = 4096 766-769 -> 703-707 us against the 32-deep
                // 4/4 tile (the fastest ring of that tile when group 0 alone
                // issues the DMA: 2 to 7 weight stages measured)
                if (avg < 192) launch_pp_persistent<192, 256, MODE, 64, 3, 2, true>(p, stream);
                else launch_pp_persistent<192, 256, MODE, 64, 3, 2, false, kFlagSplitDma>(p, stream);
                break;
            case 128: launch_pp_persistent<128, 256, MODE, 64, 4, 2>(p, stream); break;
            case 64: launch_pp_persistent<64, 256, MODE, 64, 3>(p, stream); break;
            default: launch_pp_persistent<32, 128, MODE, 64, 4>(p, stream); break;
        }
    }
    prof_end(stream, kid);
}

hipError_t launch_scatter_ffn(const uint16_t *x, const uint16_t *w1, const uint16_t *w3, const uint16_t *w2,
                              const float *topk_weights, const int32_t *expert_offsets, const int32_t *slot_src,
                              int S, int D, int F, int E, int k, uint16_t *out, uint16_t *saved, void *workspace,
                              bool atomic, hipStream_t stream) {
    const FfnPlan pl = ffn_plan(S, D, F, E, k, atomic);
    char *ws = reinterpret_cast<char *>(workspace);
    int4 *tiles_up = reinterpret_cast<int4 *>(ws + pl.tiles_up_off);
    int4 *tiles_down = reinterpret_cast<int4 *>(ws + pl.tiles_down_off);
    uint16_t *h = reinterpret_cast<uint16_t *>(ws + pl.h_off);
    float *acc = reinterpret_cast<float *>(ws + pl.acc_off);
    const int N = S * k;
    const size_t n4 = (size_t)S * D / 4;

    uint32_t *order_up = reinterpret_cast<uint32_t *>(ws + pl.order_up_off);
    uint32_t *order_down = reinterpret_cast<uint32_t *>(ws + pl.order_down_off);
    const int64_t avg = (int64_t)N / E;
    TileTableArgs ta{};
    ta.bm[0] = pl.bm_up;
    ta.bm[1] = pl.bm_down;
    ta.n_mtiles[0] = pl.n_mtiles_up;
    ta.n_mtiles[1] = pl.n_mtiles_down;
    ta.n_ntiles[0] = pl.n_ntiles_up;
    ta.n_ntiles[1] = pl.n_ntiles_down;
    ta.tiles[0] = tiles_up;
    ta.tiles[1] = tiles_down;
    ta.order[0] = order_up;
    ta.order[1] = order_down;
    int *valid_counts = reinterpret_cast<int *>(ws + pl.counts_off);
    ta.valid[0] = valid_counts;
    ta.valid[1] = valid_counts + 1;
    // the gate+up GEMM claims its tiles from per-XCD queues
    int *queue_up = reinterpret_cast<int *>(ws + pl.queue_off);
    ta.queue[0] = queue_up;
    ta.queue[1] = nullptr;
    ta.split[0] = (pl.bm_up == 256 && avg < kUpPlainRows);
    launch_tile_table(expert_offsets, E, N, ta, stream);
    if (atomic) {
        prof_begin(stream, kKAccZero);
        acc_zero_kernel<<<grid_for(n4, 256 * 4), 256, 0, stream>>>(reinterpret_cast<float4 *>(acc), n4);
        prof_end(stream, kKAccZero);
    }

    GemmParams p{};
    p.slot_src = slot_src;
    p.gate = topk_weights;
    p.topk = k;
    p.A_rows = S;

    // gate + up: A = gathered token rows of x, K = D, N = F
    p.tiles = tiles_up;
    p.order = order_up;
    p.n_mtiles = pl.n_mtiles_up;
    p.A = x;
    p.B0 = w1;
    p.B1 = w3;
    // training mode: a | b and h go to the caller's buffer for the backward
    uint16_t *h_rows = saved ? saved + (size_t)N * 2 * F : h;
    p.C = saved ? static_cast<void *>(saved) : static_cast<void *>(h);
    p.C2 = h_rows;
    p.M = N;
    p.N = F;
    p.K = D;
    p.valid_mtiles = valid_counts;
    p.queue = queue_up;
    if (saved) launch_gemm<kGateUpSave>(pl.bm_up, avg, p, stream);
    else launch_gemm<kGateUp>(pl.bm_up, avg, p, stream);

    // down + scatter-add (atomic) or per-route rows: A = h (slot order), K = F, N = D
    p.tiles = tiles_down;
    p.order = order_down;
    p.valid_mtiles = valid_counts + 1;
    p.queue = nullptr;
    p.n_mtiles = pl.n_mtiles_down;
    p.A = h_rows;
    p.C2 = nullptr;
    p.B0 = w2;
    p.B1 = nullptr;
    p.C = acc;
    p.N = D;
    p.K = F;
    if (atomic) {
        launch_gemm<kDown>(pl.bm_down, avg, p, stream);
        prof_begin(stream, kKFinalize);
        acc_finalize_kernel<<<grid_for(n4, 256 * 4), 256, 0, stream>>>(reinterpret_cast<const float4 *>(acc),
                                                                        reinterpret_cast<uint2 *>(out), n4);
        prof_end(stream, kKFinalize);
    } else {
        launch_gemm<kDownRows>(pl.bm_down, avg, p, stream);
        launch_combine_rows(acc, out, S, D, k, stream);
    }
    return hipGetLastError();
}

}  // namespace smoe
