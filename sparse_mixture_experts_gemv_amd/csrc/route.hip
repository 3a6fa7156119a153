// Router: H(X) = Softmax(TopK(X W_gate, k)) (ScatterMoE Guide, section
// "1. The Dynamic Routing Imbalance Dilemma", equation H(X)).
//
// Two paths, both ending in the same top-k rule (larger logit first, equal
// logits -> lower expert id) and an fp32 softmax over the k chosen logits with
// the maximum subtracted:
//
//  * E <= 16 (route_small_kernel): the router GEMM is tiny (2 S D E FLOP)
//    and the pass is bound by reading x once. A workgroup scores 64 / E
//    tokens: its 256 lanes split D into 8-column chunks, each lane holds the
//    W_gate rows of its chunk in registers and accumulates all the
//    workgroup's (token, expert) partial sums; a reduce-scatter over the wave
//    and a fixed-order sum of the four waves in LDS give the logits, and one
//    thread per token runs top-k and softmax. No logits buffer.
//  * larger E: logits = x W_gate on bf16 MFMA with the ping-pong LDS-DMA GEMM
//    (plain-rows mode), split over K so that a few thousand tokens still
//    fill the GPU; every split writes its partial logits to the workspace and
//    topk_softmax_kernel adds the splits in a fixed order (deterministic),
//    16 lanes per token.
#include <math.h>

#include "gemm.hpp"
#include "gemm_pp.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

constexpr int kRouteMaxE = 256;
constexpr int kRouteBM = 128;      // token rows per split-K logits tile
constexpr int kRouteBlocks = 256;  // splits are chosen to give about this many workgroups
constexpr int kRouteStages = 3;  // logits ring depth (DS-V3 shape: 33.7 -> 29.5 us against 2)
constexpr int kRouteMaxK = 16;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int E>
__global__ __launch_bounds__(256) void route_small_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ wg, int S, int D, int k,
                                                          int32_t *__restrict__ ids, float *__restrict__ weights) {
    static_assert(E % 8 == 0 && E <= 16, "small-E path");
    constexpr int TB = 64 / E;   // tokens per workgroup
    constexpr int V = TB * E;    // partial sums per lane: V = 64, value t E + e
    constexpr int EC = E / 8;    // 16-byte chunks per W_gate row
    __shared__ float s_part[4][V];
    __shared__ float s_logit[V];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = blockIdx.x * TB;
    float acc[V];
#pragma unroll
    for (int v = 0; v < V; ++v) acc[v] = 0.f;
    // chunk c covers columns 8 c .. 8 c + 7 of D; the 256 lanes of the
    // workgroup take consecutive chunks, so every token row is read once,
    // 1 KB contiguous per wave and load
    for (int c = wave * 64 + lane; c < D / 8; c += 256) {
        const int d0 = c * 8;
        uint4 w[8][EC];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
#pragma unroll
            for (int q = 0; q < EC; ++q)
                w[rr][q] = *reinterpret_cast<const uint4 *>(wg + (size_t)(d0 + rr) * E + q * 8);
        uint4 xv[TB];
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const int tt = min(t0 + t, S - 1);  // rows past S repeat a valid row, never written
            xv[t] = *reinterpret_cast<const uint4 *>(x + (size_t)tt * D + d0);
        }
#pragma unroll
        for (int t = 0; t < TB; ++t) {
            const uint32_t xw[4] = {xv[t].x, xv[t].y, xv[t].z, xv[t].w};
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const float xf = (rr & 1) ? bf16_hi(xw[rr >> 1]) : bf16_lo(xw[rr >> 1]);
#pragma unroll
                for (int q = 0; q < EC; ++q) {
                    const uint32_t ww[4] = {w[rr][q].x, w[rr][q].y, w[rr][q].z, w[rr][q].w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float wf = (e & 1) ? bf16_hi(ww[e >> 1]) : bf16_lo(ww[e >> 1]);
                        acc[t * E + q * 8 + e] = fmaf(xf, wf, acc[t * E + q * 8 + e]);
                    }
                }
            }
        }
    }
    // Reduce-scatter over the 64 lanes: at distance d the lane with bit d set
    // keeps the upper half of its values and sends the lower half, so after
    // six steps lane l holds the complete wave sum of value l.
#pragma unroll
    for (int d = 32, n = V; d >= 1; d >>= 1, n >>= 1) {
        const bool upper = (lane & d) != 0;
#pragma unroll
        for (int i = 0; i < n / 2; ++i) {
            const float lo = acc[i], hi = acc[i + n / 2];
            const float recv = __shfl_xor(upper ? lo : hi, d);
            acc[i] = (upper ? hi : lo) + recv;
        }
    }
    static_assert(V == 64, "one value per lane after the reduce-scatter");
    s_part[wave][lane] = acc[0];
    __syncthreads();
    if (threadIdx.x < V) {
        const int v = threadIdx.x;
        s_logit[v] = ((s_part[0][v] + s_part[1][v]) + s_part[2][v]) + s_part[3][v];
    }
    __syncthreads();
    // top-k + softmax, one thread per token
    if (threadIdx.x < TB && t0 + (int)threadIdx.x < S) {
        const int t = t0 + threadIdx.x;
        const float *lg = s_logit + threadIdx.x * E;
        unsigned taken = 0;
        float top[kRouteMaxK];
        int topi[kRouteMaxK];
        for (int j = 0; j < k; ++j) {
            float bv = -INFINITY;
            int bi = -1;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                if (!((taken >> e) & 1u) && (bi < 0 || lg[e] > bv)) {
                    bv = lg[e];
                    bi = e;
                }
            }
            taken |= 1u << bi;
            top[j] = bv;
            topi[j] = bi;
        }
        const float m = top[0];
        float z = 0.f;
        for (int j = 0; j < k; ++j) z += expf(top[j] - m);
        for (int j = 0; j < k; ++j) {
            ids[(size_t)t * k + j] = topi[j];
            weights[(size_t)t * k + j] = expf(top[j] - m) / z;
        }
    }
}

// logits = sum over `nsplit` partial sums [nsplit][S][E] (fixed order), then
// top-k (descending, ties to the lower expert id) and the softmax over the k
// selected logits. A group of 16 lanes serves one token (4 tokens per wave):
// lane l holds experts 4 l + c + 64 j (c < 4, j < 4), loaded as 16-byte
// pieces (E is a multiple of 8, so a piece lies wholly below E or wholly past
// it), so each round of the selection is a scan of 16 register values in
// ascending expert order and a 4-step reduction within the group.
constexpr int kTopkLanes = 16;

__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ partial, int nsplit, int S, int E,
                                                           int k, int32_t *__restrict__ ids,
                                                           float *__restrict__ weights) {
    constexpr int G = kTopkLanes, NJ = kRouteMaxE / (4 * G);  // 4 pieces of 4 experts per lane
    const int l = threadIdx.x & (G - 1);
    const int s = blockIdx.x * (256 / G) + (threadIdx.x / G);
    const int sr = min(s, S - 1);  // groups past S read a valid row and write nothing
    float v[NJ][4];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int c = 0; c < 4; ++c) v[j][c] = 0.f;
    // splits are added in order; four splits of loads are in flight at a time
    for (int q0 = 0; q0 < nsplit; q0 += 4) {
        float4 t[4][NJ];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                const int e = 4 * l + 64 * j;
                t[u][j] = (q0 + u < nsplit && e < E)
                              ? *reinterpret_cast<const float4 *>(partial + ((size_t)(q0 + u) * S + sr) * E + e)
                              : make_float4(0.f, 0.f, 0.f, 0.f);
            }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                v[j][0] += t[u][j].x;
                v[j][1] += t[u][j].y;
                v[j][2] += t[u][j].z;
                v[j][3] += t[u][j].w;
            }
    }
    unsigned taken = 0;  // bit 4 j + c: expert 4 l + c + 64 j already selected, or past E
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        if (4 * l + 64 * j >= E) taken |= 15u << (4 * j);
    float top[kRouteMaxK];
    int topi[kRouteMaxK];
#pragma unroll
    for (int r = 0; r < kRouteMaxK; ++r) {
        top[r] = -INFINITY;
        topi[r] = 0;
        if (r < k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < NJ; ++j)  // experts ascend with (j, c): an equal later value never wins
#pragma unroll
                for (int c = 0; c < 4; ++c)
                    if (!((taken >> (4 * j + c)) & 1u) && v[j][c] > bv) {
                        bv = v[j][c];
                        bi = 4 * l + c + 64 * j;
                    }
#pragma unroll
            for (int d = G / 2; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (bi < E && ((bi >> 2) & (G - 1)) == l) taken |= 1u << (4 * (bi >> 6) + (bi & 3));
            top[r] = bv;
            topi[r] = bi;
        }
    }
    const float m = top[0];
    float z = 0.f;
#pragma unroll
    for (int r = 0; r < kRouteMaxK; ++r)
        if (r < k) z += expf(top[r] - m);
#pragma unroll
    for (int r = 0; r < kRouteMaxK; ++r) {
        if (r < k && l == r && s < S) {
            ids[(size_t)s * k + r] = topi[r];
            weights[(size_t)s * k + r] = expf(top[r] - m) / z;
        }
    }
}

// Split-K router logits: block (m tile, split) computes rows [kRouteBM mt, +kRouteBM)
// x all E columns over k-steps [split KT / n, (split + 1) KT / n) and stores
// its partial sums to partial[split].
template <int BN>
__global__ __launch_bounds__(512) void route_logits_kernel(GemmParams p, int nsplit, float *partial) {
    constexpr int BM = kRouteBM, BK = 64, ST = kRouteStages;
    __shared__ __attribute__((aligned(1024))) char smem[PPGeom<BM, BN, kLogits, BK, ST>::SMEM];
    const int mt = blockIdx.x / nsplit, split = blockIdx.x % nsplit;
    const int KT = p.K / BK;
    const int kb = KT * split / nsplit, ke = KT * (split + 1) / nsplit;
    if (kb >= ke) return;
    p.C = partial + (size_t)split * p.M * p.N;
    pp_tile<BM, BN, kLogits, BK, ST>(p, smem, mt, 0, kb, ke);
}

struct RoutePlan {
    int nsplit;
    size_t ws_bytes;
};

static RoutePlan route_plan(int64_t S, int64_t D, int64_t E) {
    RoutePlan pl{1, 0};
    if (E <= 16) return pl;
    // about 256 workgroups: measured on DS-V3 (E = 256, S = 4096), 8 splits take
    // 24.7 + 18.9 us against 32.1 + 24.1 us with 16 (half the partial-logit
    // round trip) and 32.7 + 16.4 us with 4 (too few workgroups for the GEMM)
    const int64_t mtiles = (S + kRouteBM - 1) / kRouteBM, KT = D / 64;
    int64_t ns = (kRouteBlocks + mtiles - 1) / mtiles;
    if (ns > KT) ns = KT;
    if (ns < 1) ns = 1;
    pl.nsplit = (int)ns;
    pl.ws_bytes = align_up((size_t)ns * (size_t)S * (size_t)E * sizeof(float));
    return pl;
}

// Workspace bound that does not depend on D: the split count is at most
// ceil(256 / m tiles) (the plan may clamp it further to D / 64).
size_t route_ws_bytes(int64_t S, int64_t E) {
    if (E <= 16) return 0;
    const int64_t mtiles = (S + kRouteBM - 1) / kRouteBM;
    const int64_t ns = mtiles > 0 ? (kRouteBlocks + mtiles - 1) / mtiles : 1;
    return align_up((size_t)ns * (size_t)S * (size_t)E * sizeof(float));
}

hipError_t launch_route(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, int k, int32_t *topk_ids,
                        float *topk_weights, void *workspace, hipStream_t stream) {
    if (E <= 16) {
        const int blocks = (S + 64 / E - 1) / (64 / E);
        prof_begin(stream, kKRouteLogits);
        if (E == 8) route_small_kernel<8><<<blocks, 256, 0, stream>>>(x, w_gate, S, D, k, topk_ids, topk_weights);
        else route_small_kernel<16><<<blocks, 256, 0, stream>>>(x, w_gate, S, D, k, topk_ids, topk_weights);
        prof_end(stream, kKRouteLogits);
        return hipGetLastError();
    }
    const RoutePlan pl = route_plan(S, D, E);
    float *partial = reinterpret_cast<float *>(workspace);
    GemmParams p{};
    p.A = x;
    p.B0 = w_gate;
    p.M = S;
    p.A_rows = S;
    p.N = E;
    p.K = D;
    p.topk = 1;
    p.n_mtiles = (S + kRouteBM - 1) / kRouteBM;
    p.n_ntiles = 1;
    const int blocks = p.n_mtiles * pl.nsplit;
    prof_begin(stream, kKRouteLogits);
    if (E <= 64) route_logits_kernel<64><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    else if (E <= 128) route_logits_kernel<128><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    else route_logits_kernel<256><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    prof_end(stream, kKRouteLogits);
    prof_begin(stream, kKRouteTopk);
    topk_softmax_kernel<<<(S + 256 / kTopkLanes - 1) / (256 / kTopkLanes), 256, 0, stream>>>(
        partial, pl.nsplit, S, E, k, topk_ids, topk_weights);
    prof_end(stream, kKRouteTopk);
    return hipGetLastError();
}

}  // namespace smoe
