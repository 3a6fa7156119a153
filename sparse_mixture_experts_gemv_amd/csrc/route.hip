// Router: H(X) = Softmax(TopK(X W_gate, k)) (ScatterMoE Guide, section
// "1. The Dynamic Routing Imbalance Dilemma", equation H(X)).
//
// Two paths, both ending in the same top-k rule (larger logit first, equal
// logits -> lower expert id) and an fp32 softmax over the k chosen logits with
// the maximum subtracted:
//
//  * E <= 16 (route_small_kernel): the router GEMM is tiny (2 S D E FLOP)
//    and the pass is bound by reading x once. Each wave scores R tokens:
//    lane l owns columns d = 8 l + 512 j of D, keeps that slice of W_gate in
//    registers while it walks the R token rows, then a wave reduction gives
//    every lane all E logits and the top-k/softmax runs in registers. No
//    logits buffer.
//  * larger E: logits = x W_gate on bf16 MFMA with the ping-pong LDS-DMA GEMM
//    (plain-rows mode), split over K so that a few thousand tokens still
//    fill the GPU; every split writes its partial logits to the workspace and
//    topk_softmax_kernel adds the splits in a fixed order (deterministic),
//    one wavefront per token.
#include <math.h>

#include "gemm.hpp"
#include "gemm_pp.hpp"
#include "launch.hpp"
#include "profile.hpp"

namespace smoe {

constexpr int kRouteMaxE = 256;
constexpr int kRouteMaxK = 16;
constexpr int kSmallR = 4;  // tokens per wave in the small-E path

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

template <int E>
__global__ __launch_bounds__(256) void route_small_kernel(const uint16_t *__restrict__ x,
                                                          const uint16_t *__restrict__ wg, int S, int D, int k,
                                                          int32_t *__restrict__ ids, float *__restrict__ weights) {
    static_assert(E % 8 == 0 && E <= 16, "small-E path");
    constexpr int R = kSmallR;
    constexpr int EC = E / 8;  // 16-byte chunks per W_gate row
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int t0 = (blockIdx.x * 4 + wave) * R;
    if (t0 >= S) return;
    float acc[R][E];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) acc[r][e] = 0.f;
    for (int d0 = lane * 8; d0 < D; d0 += 512) {
        uint4 w[8][EC];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr)
#pragma unroll
            for (int c = 0; c < EC; ++c)
                w[rr][c] = *reinterpret_cast<const uint4 *>(wg + (size_t)(d0 + rr) * E + c * 8);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int t = min(t0 + r, S - 1);  // rows past S repeat a valid row, never written
            const uint4 xv = *reinterpret_cast<const uint4 *>(x + (size_t)t * D + d0);
            const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
            for (int rr = 0; rr < 8; ++rr) {
                const float xf = (rr & 1) ? bf16_hi(xw[rr >> 1]) : bf16_lo(xw[rr >> 1]);
#pragma unroll
                for (int c = 0; c < EC; ++c) {
                    const uint32_t ww[4] = {w[rr][c].x, w[rr][c].y, w[rr][c].z, w[rr][c].w};
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        const float wf = (q & 1) ? bf16_hi(ww[q >> 1]) : bf16_lo(ww[q >> 1]);
                        acc[r][c * 8 + q] = fmaf(xf, wf, acc[r][c * 8 + q]);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float v = acc[r][e];
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d);
            acc[r][e] = v;
        }
    // every lane now holds all logits; top-k + softmax (lane j writes rank j)
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int t = t0 + r;
        if (t >= S) break;
        unsigned taken = 0;
        float top[kRouteMaxK];
        int topi[kRouteMaxK];
#pragma unroll
        for (int j = 0; j < kRouteMaxK; ++j) {
            top[j] = -INFINITY;
            topi[j] = 0;
            if (j < k) {
                float bv = -INFINITY;
                int bi = 0;
                bool found = false;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    if (!((taken >> e) & 1u) && (!found || acc[r][e] > bv)) {
                        bv = acc[r][e];
                        bi = e;
                        found = true;
                    }
                }
                taken |= 1u << bi;
                top[j] = bv;
                topi[j] = bi;
            }
        }
        const float m = top[0];
        float z = 0.f;
#pragma unroll
        for (int j = 0; j < kRouteMaxK; ++j)
            if (j < k) z += expf(top[j] - m);
#pragma unroll
        for (int j = 0; j < kRouteMaxK; ++j) {
            if (j < k && lane == j) {
                ids[(size_t)t * k + j] = topi[j];
                weights[(size_t)t * k + j] = expf(top[j] - m) / z;
            }
        }
    }
}

// logits = sum over `nsplit` partial sums [nsplit][S][E] (fixed order).
__global__ __launch_bounds__(256) void topk_softmax_kernel(const float *__restrict__ partial, int nsplit, int S, int E,
                                                           int k, int32_t *__restrict__ ids,
                                                           float *__restrict__ weights) {
    const int lane = threadIdx.x & 63;
    const int s = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (s >= S) return;
    float v[kRouteMaxE / 64];
    unsigned taken = 0;
#pragma unroll
    for (int i = 0; i < kRouteMaxE / 64; ++i) {
        const int e = lane + 64 * i;
        if (e < E) {
            float sum = 0.f;
            for (int q = 0; q < nsplit; ++q) sum += partial[((size_t)q * S + s) * E + e];
            v[i] = sum;
        } else {
            v[i] = -INFINITY;
            taken |= 1u << i;
        }
    }
    float top[kRouteMaxK];
    int topi[kRouteMaxK];
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        top[j] = -INFINITY;
        topi[j] = 0;
        if (j < k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int i = 0; i < kRouteMaxE / 64; ++i) {
                const int e = lane + 64 * i;
                if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < bi))) {
                    bv = v[i];
                    bi = e;
                }
            }
#pragma unroll
            for (int d = 32; d >= 1; d >>= 1) {
                const float ov = __shfl_xor(bv, d);
                const int oi = __shfl_xor(bi, d);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if ((bi & 63) == lane) taken |= 1u << (bi >> 6);
            top[j] = bv;
            topi[j] = bi;
        }
    }
    const float m = top[0];
    float z = 0.f;
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j)
        if (j < k) z += expf(top[j] - m);
#pragma unroll
    for (int j = 0; j < kRouteMaxK; ++j) {
        if (j < k && lane == j) {
            ids[(size_t)s * k + j] = topi[j];
            weights[(size_t)s * k + j] = expf(top[j] - m) / z;
        }
    }
}

// Split-K router logits: block (m tile, split) computes rows [128 mt, +128)
// x all E columns over k-steps [split KT / n, (split + 1) KT / n) and stores
// its partial sums to partial[split].
template <int BN>
__global__ __launch_bounds__(512) void route_logits_kernel(GemmParams p, int nsplit, float *partial) {
    constexpr int BM = 128, BK = 64, ST = 2;
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
    const int64_t mtiles = (S + 127) / 128, KT = D / 64;
    int64_t ns = (512 + mtiles - 1) / mtiles;
    if (ns > KT) ns = KT;
    if (ns < 1) ns = 1;
    pl.nsplit = (int)ns;
    pl.ws_bytes = align_up((size_t)ns * (size_t)S * (size_t)E * sizeof(float));
    return pl;
}

// Workspace bound that does not depend on D: the split count is at most
// ceil(512 / m tiles) (the plan may clamp it further to D / 64).
size_t route_ws_bytes(int64_t S, int64_t E) {
    if (E <= 16) return 0;
    const int64_t mtiles = (S + 127) / 128;
    const int64_t ns = mtiles > 0 ? (512 + mtiles - 1) / mtiles : 1;
    return align_up((size_t)ns * (size_t)S * (size_t)E * sizeof(float));
}

hipError_t launch_route(const uint16_t *x, const uint16_t *w_gate, int S, int D, int E, int k, int32_t *topk_ids,
                        float *topk_weights, void *workspace, hipStream_t stream) {
    if (E <= 16) {
        const int blocks = (S + 4 * kSmallR - 1) / (4 * kSmallR);
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
    p.n_mtiles = (S + 127) / 128;
    p.n_ntiles = 1;
    p.group_m = 1;
    const int blocks = p.n_mtiles * pl.nsplit;
    prof_begin(stream, kKRouteLogits);
    if (E <= 64) route_logits_kernel<64><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    else if (E <= 128) route_logits_kernel<128><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    else route_logits_kernel<256><<<blocks, 512, 0, stream>>>(p, pl.nsplit, partial);
    prof_end(stream, kKRouteLogits);
    prof_begin(stream, kKRouteTopk);
    topk_softmax_kernel<<<(S + 3) / 4, 256, 0, stream>>>(partial, pl.nsplit, S, E, k, topk_ids, topk_weights);
    prof_end(stream, kKRouteTopk);
    return hipGetLastError();
}

}  // namespace smoe
